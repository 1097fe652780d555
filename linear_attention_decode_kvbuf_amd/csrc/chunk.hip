// Buffered decode, draft verification and buffer-only decode (one kernel).
//
// KVBuffer: IO-aware Serving for Linear Attention (pith.science page):
//  * Figure 1 caption -- decode reads the state and the request's buffer
//    blocks side by side; a full buffer is folded into the state, which goes
//    back to its slot;
//  * Figure 2 caption -- drafts go into the buffer and are checked in one
//    pass, so no per-draft copy of the state exists;
//  * abstract -- a short request never gets a state: its buffer alone
//    yields its outputs.
//
// Unrolling the recurrence from the state S0 at the last fold (positions
// 0 .. T-1 buffered since then, b_i = g_0 + ... + g_i the cumulative log-gate):
//   o_t = e^{b_t} S0^T q_t + sum_{i<=t} e^{b_t - b_i} (q_t . k_i) x_i
//   S_t = e^{b_t} S0 + sum_{i<=t} e^{b_t - b_i} k_i x_i^T
// with x_i = v_i for the linear (b = 0) and gated rules, and for the delta rule
//   x_t = u_t = beta_t (v_t - e^{b_t} S0^T k_t - sum_{i<t} e^{b_t - b_i} (k_i . k_t) u_i),
// the pseudo-value the pool stores in place of v.
//
// One workgroup of NT threads per (request, head); each thread holds RPT rows
// x 4 columns of the 64 KiB state tile (RPT 128-bit non-temporal loads) and
// stages a share of the token rows (16 threads per position, one 16-byte
// chunk each).  A wave's memory counter retires in issue order, so what is
// issued before the tile never waits for it.  Delta rule: the first two
// passes of buffered rows (and the query, key and gate) go first, so their
// scores, gate prefix sums and decay weights are formed while the tile is in
// flight.  Linear and gated rules: the tile goes right after the metadata and
// the token work waits for it (faster for verification, whose vector work
// is heavier).  The tile is consumed last, in one pass over registers.  The
// state is the only large operand; the kernel is bound by HBM bandwidth.
#include "device_common.hpp"

namespace kvbuf {
namespace {

// LDS layout in 4-byte words (shared by the launcher, for the size, and the
// kernel).  Token rows are kept as the raw bits they were loaded with (bf16
// or fp32) and converted where they are used, so that no converted copy
// occupies registers while the state tile is in flight.
struct ChunkLds {
    int pos, qr, kdr, bl, cq, ck, es, kr, vr, fw, red, sq, sk, total;
};

__host__ __device__ inline int round4(int x) { return (x + 3) & ~3; }

// io / xo: bytes per element of the key plane and of the value plane.
// NG positions are staged per pass; `fold` = the eager fold may happen in
// this launch (then m <= NG and its keys and values are the first pass's).
__host__ __device__ inline ChunkLds chunk_lds(int rule, int DK, int DV, int NQ, int RG, int NG, int cap,
                                              int m, bool fold, int io, int xo) {
    ChunkLds L;
    int o = 0;
    const bool delta = rule == KVBUF_RULE_DELTA;
    L.pos = o; o += round4(cap);                        // pool row of each buffer position
    L.qr = o; o += round4(NQ * DK * io / 4);            // queries of the new tokens (raw)
    L.kdr = o; o += delta ? round4(NQ * DK * io / 4) : 0;  // keys of the new tokens (delta rule)
    L.bl = o; o += round4(cap);                         // log-gates, then their prefix sums
    L.cq = o; o += NQ * round4(cap);                    // e^{b_t - b_i} scale (q_t . k_i)
    L.ck = o; o += delta ? NQ * round4(cap) : 0;        // e^{b_t - b_i} (k_t . k_i)
    L.es = o; o += round4(NQ + 1);                      // e^{b_t} per new token; [NQ]: e^{b_{m-1}}
    const int slots = (delta || NQ == 1) ? 2 : 1;       // two pass slots for the direct-to-LDS ring
    L.kr = o; o += round4(slots * NG * DK * io / 4);    // keys of one pass of positions (raw)
    L.vr = o; o += round4(slots * NG * DV * xo / 4);    // their values (raw)
    L.fw = o; o += fold ? round4(m) : 0;                // fold weights
    // row-group partial sums; the matrix-core instance of eight queries keeps
    // one slot per wave (its two row groups summed first), which lets four of
    // its workgroups share a CU's LDS
    const bool ws = !delta && NQ == 8 && DK == 128 && DV == 128 && io == 2;
    L.red = o; o += (ws ? RG / 2 : RG) * DV * (delta ? 2 : NQ);
    L.sq = o; o += delta ? NQ * DV : 0;                 // reduced outputs before the new tokens
    L.sk = o; o += delta ? NQ * DV : 0;                 // reduced e^{b_t} S0^T k_t + buffer part
    L.total = o;
    return L;
}

// S0^T q for up to eight queries on the matrix cores (bf16, d_k = d_v = 128,
// 256 threads: thread t holds rows 16 (t / 32) + j, j < 16, columns
// 4 (t % 32) .. + 3 of the tile).  Wave w multiplies its 32 rows with
// v_mfma_f32_16x16x16_bf16: K = 16 = four lane groups g of four rows, B[k][n]
// = S[32w + 16 (g / 2) + 4 q + i][64 (g % 2) + 4 n + e] straight from the
// state registers (component e of s[4q + i]), M = 16 = two column halves x
// eight queries, A[8 h + d][k] = q_d[row of k] where g % 2 = h and 0 otherwise.
// The fp32 state goes in as two bf16 terms, hi = bf16(S) and lo = bf16(S -
// hi), so each product is exact and S is represented to about 2^-17 of its
// size; the bf16 queries are exact.  The wave's partial sums over its 32 rows
// are added (times scale e^{b_t}) into the wave's slot of `red` (RGS slots per
// query: the wave's own, or that of its first row group, 2w), which already
// holds the wave's value sums.
template <int DK, int DV, int RG, int RGS>
__device__ __forceinline__ void state_products_mfma(const f4 (&s)[16], const bf16_bits* qr, float* red,
                                                    const float* es, float scale, int n, int tid) {
    typedef short s4 __attribute__((ext_vector_type(4)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    const int w = tid >> 6, l = tid & 63, g = l >> 4, nn = l & 15;
    // A operands, one per quad of rows
    s4 a[4];
    const int da = l & 7;
    const bool live_a = ((g & 1) == ((l & 15) >> 3)) && da < n;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int row0 = 32 * w + 16 * (g >> 1) + 4 * q;
        a[q] = live_a ? *reinterpret_cast<const s4*>(qr + da * DK + row0) : s4{0, 0, 0, 0};
    }
    f4 d[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        d[e] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f2 x01 = {s[4 * q][e], s[4 * q + 1][e]};
            const f2 x23 = {s[4 * q + 2][e], s[4 * q + 3][e]};
            const uint32_t h01 = __builtin_bit_cast(uint32_t, __builtin_convertvector(x01, bf2));
            const uint32_t h23 = __builtin_bit_cast(uint32_t, __builtin_convertvector(x23, bf2));
            const f2 r01 = x01 - f2{__uint_as_float(h01 << 16), __uint_as_float(h01 & 0xffff0000u)};
            const f2 r23 = x23 - f2{__uint_as_float(h23 << 16), __uint_as_float(h23 & 0xffff0000u)};
            const uint32_t l01 = __builtin_bit_cast(uint32_t, __builtin_convertvector(r01, bf2));
            const uint32_t l23 = __builtin_bit_cast(uint32_t, __builtin_convertvector(r23, bf2));
            const s4 bh = __builtin_bit_cast(s4, make_uint2(h01, h23));
            const s4 bl = __builtin_bit_cast(s4, make_uint2(l01, l23));
            d[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[q], bh, d[e], 0, 0, 0);
            d[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[q], bl, d[e], 0, 0, 0);
        }
    }
    // lane l holds D[4 g + i][nn]: query 4 (g % 2) + i, column 64 (g / 2) + 4 nn + e
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int dq = 4 * (g & 1) + i;
        if (dq < n) {
            f4* dst = reinterpret_cast<f4*>(red + (dq * RGS + (RGS == RG ? 2 * w : w)) * DV + 64 * (g >> 1) + 4 * nn);
            *dst += f4{d[0][i], d[1][i], d[2][i], d[3][i]} * (scale * es[dq]);
        }
    }
}

// Scores of one pass (16 buffer positions i0 .. i0+15) against up to eight
// bf16 queries of d_k = 128, by one wave: D[d][j] = q_d . k_{i0+j} with
// v_mfma_f32_16x16x16_bf16 over eight K-slices of 16 channels (A[m][k] =
// q_m[16 c + k] from the raw query rows, zero for m >= n; B[k][j] = the raw
// key row of position i0 + j).  bf16 products are exact in fp32.  Lane l then
// holds D[4 (l / 16) + i][l % 16] and writes the decayed, scaled, masked
// score of query 4 (l / 16) + i (l < 32) at position i0 + l % 16 to cq.
template <int DK, bool TREE, bool GATED>
__device__ __forceinline__ void scores_mfma(const bf16_bits* qr, const bf16_bits* krs, float* cq, const float* bl,
                                            const uint32_t* anc, int i0, int p, int T, int n, int ldc, float scale,
                                            int lane) {
    typedef short s4 __attribute__((ext_vector_type(4)));
    const int g = lane >> 4, j = lane & 15;
    const int m = lane & 15;
    f4 dacc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < DK / 16; ++c) {
        const s4 a = m < n ? *reinterpret_cast<const s4*>(qr + m * DK + 16 * c + 4 * g) : s4{0, 0, 0, 0};
        const s4 b = *reinterpret_cast<const s4*>(krs + j * DK + 16 * c + 4 * g);
        dacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, dacc, 0, 0, 0);
    }
    const int i = i0 + j;
    const int ic = min(i, T - 1);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int d = 4 * g + r;
        if (g < 2 && d < n && i < T) {
            const int t = p + d;
            const bool seen = TREE ? (i < p || ((anc[TREE ? d : 0] >> (i - p)) & 1u)) : i <= t;
            cq[d * ldc + i] = seen ? (GATED ? exp_gate(bl[t] - bl[ic]) : 1.0f) * scale * dacc[r] : 0.f;
        }
    }
}

// TREE: the new tokens are tree drafts (parent array); otherwise a chain.
template <int RULE, int DK, int DV, int NQ, typename IO, bool TREE>
__global__ __launch_bounds__((Geo<DK, DV>::NT)) void chunk_kernel(TileParams P) {
    using G = Geo<DK, DV>;
    constexpr int NT = G::NT, TPR = G::TPR, RG = G::RG, RPT = G::RPT;
    constexpr int E = DK / 16, EV = DV / 16;
    constexpr int NG = NT / 16;               // positions per staging pass
    constexpr int NQR = (NQ + NG - 1) / NG;   // query chunks per thread
    constexpr bool DELTA = RULE == KVBUF_RULE_DELTA;
    constexpr bool GATED = RULE != KVBUF_RULE_LINEAR;
    using XIO = typename std::conditional<DELTA, float, IO>::type;
    // four or eight bf16 queries of d = 128: the scores and the state products
    // run on the matrix cores, and the value sums go straight to LDS
    constexpr bool MF = !DELTA && NQ >= 4 && DK == 128 && DV == 128 && std::is_same<IO, bf16_bits>::value;
    // eight queries: one slot of `red` per wave and query (its two row groups
    // summed first), so that four workgroups share a CU's LDS
    constexpr bool WS = MF && NQ == 8;
    constexpr int RGS = WS ? RG / 2 : RG;  // row-group slots of `red` per query
    // One new token (decode / direct with long rows) and the delta rule: the
    // keys and values (pseudo-values) of each pass are copied straight into a
    // two-slot LDS ring by direct-to-LDS loads.  The first two passes are
    // requested together (before the state tile for the delta rule), so
    // buffers of up to 2 NG positions cost one round trip; a later pass is
    // requested as soon as the pass two before it has been consumed.
    // Verification of 2-8 drafts stages its rows through registers (measured
    // faster there).
    constexpr bool DMA = DELTA || NQ == 1;
    // Linear / gated rules: the tile is requested right after the metadata,
    // ahead of the buffer's rows (the scores then wait for the tile, which
    // measured faster for verification than holding the tile back behind the
    // metadata chain).  Delta rule: the tile follows the first two passes.
    constexpr bool EARLY = !DELTA;

    extern __shared__ __attribute__((aligned(16))) float lds[];  // 16-byte rows for the LDS copies
    __shared__ unsigned s_bad;
    __shared__ int s_p;
    // Tree drafts: draft d attends to position p + e iff bit e of s_anc[d] is
    // set -- d and its ancestors (parent -1 = the buffered context).  A chain
    // (and the one token of a decode) attends to every e <= d.
    __shared__ uint32_t s_anc[TREE ? kMaxDrafts : 1];
    __shared__ float s_gnew[NQ];  // log-gates of this call's tokens

    const TileIndex ti = tile_index(P);
    const int b = ti.b;
    const int h = ti.h;
    const int tid = threadIdx.x;
    const int rg = tid / TPR;
    const int c0 = (tid % TPR) * 4;
    const int gp = tid >> 4;   // position slot of this thread in a pass
    const int cl = tid & 15;   // its 1/16 chunk of a row
    const int n = P.n;
    const int cap = P.block_size * P.blocks_per_req;
    const bool direct = P.mode == MODE_DIRECT;

    // ---- tile metadata (read by wave 0 only, which also updates it) -----------
    const int slot = direct ? -1 : P.slot[b];
    const ChunkLds L = chunk_lds(RULE, DK, DV, NQ, RG, NG, cap, P.m, P.fold_chunk > 0,
                                 static_cast<int>(sizeof(IO)), static_cast<int>(sizeof(XIO)));
    uint32_t* spos = reinterpret_cast<uint32_t*>(lds + L.pos);
    IO* qr = reinterpret_cast<IO*>(lds + L.qr);
    IO* kdr = reinterpret_cast<IO*>(lds + L.kdr);
    float* bl = lds + L.bl;
    float* cq = lds + L.cq;
    float* ck = lds + L.ck;
    float* es = lds + L.es;
    IO* krs = reinterpret_cast<IO*>(lds + L.kr);
    XIO* vrs = reinterpret_cast<XIO*>(lds + L.vr);
    float* fw = lds + L.fw;
    int p0 = 0, blk = 0;
    int par = -1;  // tree drafts: parent of draft tid
    if (tid < 64) {  // the occupancy, the table row (and the parents) in one round trip
        p0 = load_occupancy(P, b, h);
        blk = load_table_row(P, b, h, tid);
        if (TREE && tid < n) par = P.parent[static_cast<size_t>(b) * n + tid];
    }
    f4 s[RPT];
    if constexpr (EARLY) {
        __builtin_amdgcn_sched_barrier(0);  // the metadata loads go first
        const bool present = slot >= 0 && slot < P.num_slots;
        load_tile<RPT, DK, DV>(s, present ? P.state + (static_cast<size_t>(slot) * P.H + h) * DK * DV : P.state,
                               present, rg, c0);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (tid < 64) {
        unsigned bad = stage_row_from(P, h, (p0 < 0 || p0 > cap) ? -1 : p0 + n, spos, tid, blk);
        if (slot >= P.num_slots) bad |= KVBUF_DEVERR_SLOT;
        if constexpr (TREE) {
            const bool bad_par = tid < n && (par < -1 || par >= tid);  // parents precede children
            if (__ballot(bad_par)) bad |= KVBUF_DEVERR_ACCEPT;
            // ancestor mask of draft `tid` by pointer doubling: after a round
            // with span s, anc holds the draft and its ancestors less than 2s
            // levels up and `up` the one 2s levels up (-1: past the root), so
            // three rounds cover the deepest path of kMaxDrafts drafts (a tile
            // with invalid parents is skipped, whatever its masks)
            const bool mine = tid < n && !bad_par;
            uint32_t anc = mine ? 1u << tid : 0u;
            int up = mine ? par : -1;
#pragma unroll
            for (int span = 1; span < kMaxDrafts; span <<= 1) {
                const int src = up >= 0 ? up : 0;
                const uint32_t a = static_cast<uint32_t>(__shfl(static_cast<int>(anc), src, 64));
                const int u = __shfl(up, src, 64);
                if (up >= 0) {
                    anc |= a;
                    up = u;
                }
            }
            if (tid < n) s_anc[tid] = anc;
        }
        if (tid == 0) {
            s_bad = bad;
            s_p = p0;
        }
    }
    __syncthreads();  // spos, s_p and s_bad are complete
    if (s_bad) {
        report(P, s_bad);
        return;  // the tile is skipped and its metadata left unchanged
    }
    const int p = s_p;  // occupancy before this call
    const bool has_state = slot >= 0;
    const int T = p + n;                       // positions touched by this call
    const bool fold = P.fold_chunk > 0 && has_state && T >= P.m;  // launcher: fold_chunk >= m

    const int ldc = round4(cap);

    const size_t in_row = static_cast<size_t>(b) * n * P.H + h;  // (b, new token 0, h)
    TileTokens<DK, DV, IO, XIO> tok;
    tok.kpool = static_cast<const IO*>(P.key);
    tok.xpool = static_cast<const XIO*>(P.value);
    tok.gpool = P.gate;
    tok.pos = spos;
    tok.H = P.H;
    tok.p = p;
    tok.kin = static_cast<const IO*>(P.k) + in_row * DK;
    tok.vin = static_cast<const IO*>(P.v) + in_row * DV;
    tok.gin = GATED ? P.g + in_row : nullptr;
    tok.in_stride_k = static_cast<size_t>(P.H) * DK;
    tok.in_stride_v = static_cast<size_t>(P.H) * DV;
    IO* kpool = static_cast<IO*>(P.key);
    XIO* xpool = static_cast<XIO*>(P.value);

    // ---- 1. token loads of the first pass, then the state tile ----------------
    // direct-to-LDS copies of the positions i0 .. i0+NG-1 into ring rows
    // row0 .. row0+NG-1: each wave copies NG / (NT / 64) of them
    auto dma_pass = [&](int i0, int row0) {
        constexpr int RW = NG / (NT / 64);
        const int w = tid >> 6;
        const int lane = tid & 63;
        const int r0 = w * RW;
        const int nk = max(0, min(RW, T - (i0 + r0)));
        // values of every position; delta rule: pseudo-values of buffered positions only
        const int nx = max(0, min(RW, (DELTA ? p : T) - (i0 + r0)));
        lds_copy_rows<DK * static_cast<int>(sizeof(IO))>(
            reinterpret_cast<char*>(krs + (row0 + r0) * DK), nk,
            [&](int r) { return reinterpret_cast<const char*>(tok.key(i0 + r0 + r)); }, lane);
        lds_copy_rows<DV * static_cast<int>(sizeof(XIO))>(
            reinterpret_cast<char*>(vrs + (row0 + r0) * DV), nx, [&](int r) {
                const int i = i0 + r0 + r;
                if constexpr (DELTA) return reinterpret_cast<const char*>(tok.pooled_value(i));
                else return reinterpret_cast<const char*>(i < p ? tok.pooled_value(i) : tok.new_value(i - p));
            }, lane);
    };
    if constexpr (DMA) {
        dma_pass(0, 0);
        if (T > NG) dma_pass(NG, NG);
        __builtin_amdgcn_sched_barrier(0);  // the copies go first
    }
    // this call's queries, and its keys (and values, linear / gated rules) for
    // the appends.  The token loads below are issued with no branch between
    // them, from clamped indices (draft n - 1 and position T - 1 exist: n >= 1);
    // every use of a slot past the end is guarded (d < n, i < T).  Loads under
    // per-lane branches each ended with a wait for the counter to drain, which
    // put them a round trip apart.
    RawChunk<IO, E> qraw[NQR], kdraw[NQR];
    RawChunk<IO, EV> vdraw[DELTA ? 1 : NQR];
#pragma unroll
    for (int r = 0; r < NQR; ++r) {
        const int d = min(gp + NG * r, n - 1);
        qraw[r].load(static_cast<const IO*>(P.q) + (in_row + d * P.H) * DK + cl * E);
        kdraw[r].load(tok.kin + d * tok.in_stride_k + cl * E);
        if constexpr (!DELTA) vdraw[r].load(tok.new_value(d) + cl * EV);
    }
    float graw = 0.f;  // log-gate of position tid
    if constexpr (GATED) {
        const int i = min(tid, T - 1);
        graw = *(i < p ? tok.gpool + tok.slot_index(i) : tok.gin + static_cast<size_t>(i - p) * P.H);
    }
    // delta rule, one new token: its value and step size for this thread's
    // column (step 6), loaded with the rest rather than after the reductions;
    // the value is kept as loaded and converted where it is used (converting
    // here would wait for it, and with it for every copy and load above,
    // before the state tile is requested)
    constexpr bool PRE = DELTA && NQ == 1;
    IO vpre{};
    float bpre = 0.f;
    if constexpr (PRE) {
        static_assert(NT >= DV, "one column per thread");
        vpre = tok.new_value(0)[min(tid, DV - 1)];  // (columns c = tid < DV use it)
        bpre = P.beta[in_row];
    }
    RawChunk<IO, E> kr;
    RawChunk<XIO, EV> xr;
    // (the position clamped to T - 1 as above: stage_pass uses i < T only)
    auto load_pass = [&](int i0) {
        const int i = min(i0 + gp, T - 1);
        kr.load(tok.key(i) + cl * E);
        if constexpr (DELTA) {
            xr.zero();
            if (i < p) xr.load(tok.pooled_value(i) + cl * EV);
        } else {
            xr.load((i < p ? tok.pooled_value(i) : tok.new_value(i - p)) + cl * EV);
        }
    };
    if constexpr (!DMA) load_pass(0);
    __builtin_amdgcn_sched_barrier(0);  // keep every token load ahead of the state loads

    if constexpr (!EARLY)
        load_tile<RPT, DK, DV>(s, has_state ? P.state + (static_cast<size_t>(slot) * P.H + h) * DK * DV : P.state,
                               has_state, rg, c0);
    if constexpr (DMA && !EARLY) {
        // Everything but the RPT state loads has landed (a wave's loads retire
        // in issue order), so the copied rows are in LDS once the barrier
        // below is passed.  gfx9 encoding of vmcnt(RPT), other counters free.
        static_assert(RPT < 64, "vmcnt field");
        __builtin_amdgcn_s_waitcnt((RPT & 15) | ((RPT >> 4) << 14) | 0x0F70);
        __builtin_amdgcn_sched_barrier(0);
    } else if constexpr (DMA) {
        wait_lds_copies();  // the copies follow the tile here
    }

    // ---- 2. token data to LDS as raw bits; appends from the same registers -----
#pragma unroll
    for (int r = 0; r < NQR; ++r) {
        const int d = gp + NG * r;
        if (d < n) {
            qraw[r].store(qr + d * DK + cl * E);
            if constexpr (DELTA) kdraw[r].store(kdr + d * DK + cl * E);
        }
    }
    // log-gates of every position; the new tokens' are kept aside for their
    // append at the end (a store here would hold up the next barrier, a
    // register would be live through the whole kernel)
    if (GATED && tid < T) {
        bl[tid] = graw;
        if (tid >= p) s_gnew[tid - p] = graw;
    }
    for (int i = NT + tid; GATED && i < T; i += NT) {  // long buffers only
        const float gi = tok.gate(i);
        bl[i] = gi;
        if (i >= p) s_gnew[i - p] = gi;
    }
    auto stage_pass = [&](int i0) {
        const int i = i0 + gp;
        if (i < T) {
            kr.store(krs + gp * DK + cl * E);
            xr.store(vrs + gp * DV + cl * EV);
            if (i >= p) {  // append this call's tokens
                kr.store(kpool + tok.slot_index(i) * DK + cl * E);
                if constexpr (!DELTA) xr.store(xpool + tok.slot_index(i) * DV + cl * EV);
            }
        }
    };
    if constexpr (DMA) {
        // append this call's keys (and values) from the registers they were
        // loaded into; delta-rule pseudo-values are appended once formed
#pragma unroll
        for (int r = 0; r < NQR; ++r) {
            const int d = gp + NG * r;
            if (d < n) {
                kdraw[r].store(kpool + tok.slot_index(p + d) * DK + cl * E);
                if constexpr (!DELTA) vdraw[r].store(xpool + tok.slot_index(p + d) * DV + cl * EV);
            }
        }
    } else {
        stage_pass(0);
    }
    __syncthreads();

    // ---- 3. cumulative log-gates (wave 0), decay weights of S0 -----------------
    if (tid < 64) {
        if constexpr (GATED) {
            // tree drafts: every draft's log-gate, read by every lane (the
            // same LDS word for all lanes) before the prefix overwrites it
            float gd[TREE ? kMaxDrafts : 1];
            if constexpr (TREE) {
#pragma unroll
                for (int e = 0; e < kMaxDrafts; ++e) gd[e] = e < n ? bl[p + e] : 0.0f;
            }
            gate_prefix(bl, T, tid, [&](int i) { return bl[i]; });
            if constexpr (TREE) {
                // tree drafts: the decay of draft d runs along its own path,
                // b_{p+d} = b_{p-1} + the log-gates of d and its ancestors
                const uint32_t anc = tid < n ? s_anc[tid] : 0u;
                float acc = p > 0 ? bl[p - 1] : 0.0f;
#pragma unroll
                for (int e = 0; e < kMaxDrafts; ++e)
                    if (e < n && ((anc >> e) & 1u)) acc += gd[e];
                if (tid < n) bl[p + tid] = acc;
            }
        } else {
            for (int i = tid; i < T; i += 64) bl[i] = 0.0f;
        }
        if (tid < n) es[tid] = GATED ? exp_gate(bl[p + tid]) : 1.0f;
        if (fold && tid == 0) es[NQ] = GATED ? exp_gate(bl[P.m - 1]) : 1.0f;
    }
    __syncthreads();

    // ---- 4. per pass: scores of its positions, weighted value sums -------------
    f4 acc[MF ? 1 : NQ];
    f4 acck[DELTA ? NQ : 1];
#pragma unroll
    for (int d = 0; d < (MF ? 1 : NQ); ++d) {
        acc[d] = f4{0.f, 0.f, 0.f, 0.f};
        if constexpr (DELTA) acck[d] = f4{0.f, 0.f, 0.f, 0.f};
    }
    const int tacc = DELTA ? p : T;  // positions whose values enter the sums here
    for (int i0 = 0; i0 < T; i0 += NG) {
        const int rbase = DMA ? ((i0 / NG) & 1) * NG : 0;  // ring slot of this pass's rows
        if (i0 > 0) {
            if constexpr (DMA) {
                if (i0 >= 2 * NG) {
                    // requested at the end of the pass two before this one;
                    // those copies follow the state loads, so this waits for them
                    wait_lds_copies();
                    __syncthreads();
                }
            } else {
                // Later passes (buffers longer than NG positions): these loads
                // follow the state loads, so they wait for them.
                __syncthreads();  // the previous pass's rows are consumed
                load_pass(i0);
                stage_pass(i0);
                __syncthreads();
            }
        }
        const int i = i0 + gp;
        const int ic = min(i, T - 1);
        if constexpr (MF) {
            // wave 0: the pass's 16 positions x the queries on the matrix cores
            if (tid < 64)
                scores_mfma<DK, TREE, GATED>(qr, krs + rbase * DK, cq, bl, s_anc, i0, p, T, n, ldc, P.scale, tid);
        }
        RawChunk<IO, E> kc;
        if (!MF) kc.load(krs + (rbase + gp) * DK + cl * E);
#pragma unroll
        for (int d = 0; d < NQ; ++d) {
            if (!MF && d < n) {
                const int t = p + d;
                // the buffered context, then the new tokens on d's path
                const bool seen = TREE ? (i < p || (i < T && ((s_anc[TREE ? d : 0] >> (i - p)) & 1u))) : i <= t;
                RawChunk<IO, E> qc;
                qc.load(qr + d * DK + cl * E);
                const float dot = group16_sum(chunk_dot(qc, kc));
                const float wq = seen ? (GATED ? exp_gate(bl[t] - bl[ic]) : 1.0f) * P.scale * dot : 0.f;
                if (cl == 0 && i < T) cq[d * ldc + i] = wq;
                if constexpr (DELTA) {
                    qc.load(kdr + d * DK + cl * E);
                    const float dk = group16_sum(chunk_dot(qc, kc));
                    const float wk = (TREE ? (seen && i != t) : i < t) ? (GATED ? exp_gate(bl[t] - bl[ic]) : 1.0f) * dk : 0.f;
                    if (cl == 0 && i < T) ck[d * ldc + i] = wk;
                }
            }
        }
        __syncthreads();
        // weighted sums: row group rg takes the pass positions ii = rg, rg+RG, ...
        const int cnt = min(NG, tacc - i0);
        if constexpr (MF) {
            // one query at a time, straight into this wave's slot of `red`
            // (no accumulator stays live next to the tile)
            float* red = lds + L.red;
            // (WS: lanes l and l + 32 of a wave hold the same columns of its
            // two row groups; their sums are added and the wave's slot updated)
#pragma unroll
            for (int d = 0; d < NQ; ++d) {
                if (d < n) {
                    f4 a = f4{0.f, 0.f, 0.f, 0.f};
                    for (int ii = rg; ii < cnt; ii += RG)
                        a += cq[d * ldc + i0 + ii] * load4(vrs + (rbase + ii) * DV + c0);
                    if constexpr (WS) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) a[e] += __shfl_xor(a[e], 32, 64);
                    }
                    if (!WS || (tid & 32) == 0) {
                        f4* own = reinterpret_cast<f4*>(red + (d * RGS + (WS ? tid >> 6 : rg)) * DV + c0);
                        *own = i0 > 0 ? *own + a : a;
                    }
                }
            }
        } else {
            for (int ii = rg; ii < cnt; ii += RG) {
                const f4 x = load4(vrs + (rbase + ii) * DV + c0);
#pragma unroll
                for (int d = 0; d < NQ; ++d) {
                    if (d < n) {
                        acc[d] += cq[d * ldc + i0 + ii] * x;
                        if constexpr (DELTA) acck[d] += ck[d * ldc + i0 + ii] * x;
                    }
                }
            }
        }
        if constexpr (DMA) {
            if (i0 + 2 * NG < T) {
                __syncthreads();  // every wave is done with this slot
                dma_pass(i0 + 2 * NG, rbase);
            }
        }
    }
    if (fold && T > (DMA ? 2 * NG : NG)) {
        // Rare: the buffer outgrew the passes still staged before an eager
        // fold (only after deferred-policy calls).  The m positions to fold
        // are all in the pool (p >= m); stage them again.
        __syncthreads();
        kr.zero();
        xr.zero();
        if (gp < P.m) {
            kr.load(tok.key(gp) + cl * E);
            xr.load(tok.pooled_value(gp) + cl * EV);
            kr.store(krs + gp * DK + cl * E);
            xr.store(vrs + gp * DV + cl * EV);
        }
    }
    if (fold && tid < P.m) fw[tid] = GATED ? exp_gate(bl[P.m - 1] - bl[tid]) : 1.0f;

    // The new tokens' log-gates go to the pool after the last barrier (a
    // barrier waits for the stores before it).
    auto append_gates = [&]() {
        if (GATED && tid < n) P.gate[tok.slot_index(p + tid)] = s_gnew[tid];
    };

    // ---- 5. the state tile: S^T q (and S^T k), reduced over row groups --------
    float* red = lds + L.red;
    const size_t outp = in_row * DV;  // output element of (request, draft 0, head)
    const size_t out_stride = static_cast<size_t>(P.H) * DV;
    if constexpr (MF) {  // the value sums are in `red` already
        if (has_state) state_products_mfma<DK, DV, RG, RGS>(s, qr, red, es, P.scale, n, tid);
    }
    if constexpr (!DELTA) {
        // every query's row-group partials at once, then one reduction
#pragma unroll
        for (int d = 0; d < NQ; ++d) {
            if (!MF && d < n) {
                f4 a = acc[d];
                if (has_state) {
                    RawChunk<IO, RPT> qrow;
                    float qf[RPT];
                    qrow.load(qr + d * DK + rg * RPT);
                    qrow.to_float(qf);
                    f4 sa = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < RPT; ++j) sa += s[j] * qf[j];
                    a += sa * (P.scale * es[d]);
                }
                *reinterpret_cast<f4*>(red + (d * RGS + rg) * DV + c0) = a;
            }
        }
        __syncthreads();
        append_gates();
        for (int idx = tid; idx < n * DV; idx += NT) {
            const int d = idx / DV;
            const int c = idx - d * DV;
            float sum = 0.f;
#pragma unroll
            for (int g2 = 0; g2 < RGS; ++g2) sum += red[(d * RGS + g2) * DV + c];
            store_out(P, outp + d * out_stride + c, sum);
        }
    } else {
#pragma unroll
        for (int d = 0; d < NQ; ++d) {
            if (d < n) {
                f4 a = acc[d];
                f4 ak = acck[d];
                if (has_state) {
                    f4 sa = f4{0.f, 0.f, 0.f, 0.f};
                    f4 sk = f4{0.f, 0.f, 0.f, 0.f};
                    RawChunk<IO, RPT> qrow, krow;
                    float qf[RPT], kf[RPT];
                    qrow.load(qr + d * DK + rg * RPT);
                    qrow.to_float(qf);
                    krow.load(kdr + d * DK + rg * RPT);
                    krow.to_float(kf);
#pragma unroll
                    for (int j = 0; j < RPT; ++j) {
                        sa += s[j] * qf[j];
                        sk += s[j] * kf[j];
                    }
                    a += sa * (P.scale * es[d]);
                    ak += sk * es[d];
                }
                *reinterpret_cast<f4*>(red + rg * DV + c0) = a;
                *reinterpret_cast<f4*>(red + (RG + rg) * DV + c0) = ak;
                __syncthreads();
                for (int c = tid; c < DV; c += NT) {
                    float sum = 0.f, sumk = 0.f;
#pragma unroll
                    for (int g2 = 0; g2 < RG; ++g2) {
                        sum += red[g2 * DV + c];
                        sumk += red[(RG + g2) * DV + c];
                    }
                    lds[L.sq + d * DV + c] = sum;
                    lds[L.sk + d * DV + c] = sumk;
                }
                __syncthreads();  // `red` is reused by the next query; step 6 reads sq / sk
            }
        }
    }

    // ---- 6. delta rule: pseudo-values and outputs of the new tokens ------------
    if constexpr (DELTA) {
        for (int c = tid; c < DV; c += NT) {
            float u[NQ];
#pragma unroll
            for (int d = 0; d < NQ; ++d) {
                u[d] = 0.f;
                if (d < n) {
                    const int t = p + d;
                    float x = (PRE ? as_float(vpre) : load1(tok.new_value(d) + c)) - lds[L.sk + d * DV + c];
                    float o = lds[L.sq + d * DV + c];
#pragma unroll
                    for (int e = 0; e < d; ++e) x -= ck[d * ldc + p + e] * u[e];
                    x *= PRE ? bpre : P.beta[in_row + static_cast<size_t>(d) * P.H];
                    u[d] = x;
#pragma unroll
                    for (int e = 0; e <= d; ++e) o += cq[d * ldc + p + e] * u[e];
                    store_out(P, outp + d * out_stride + c, o);
                    xpool[tok.slot_index(t) * DV + c] = x;
                    if (fold && t < P.m) vrs[t * DV + c] = x;  // the new token is folded too
                }
            }
        }
        __syncthreads();
        append_gates();
    }

    // ---- 7. eager fold: the buffer reached m tokens ----------------------------
    if (fold) {
        const float e0 = es[NQ];
#pragma unroll
        for (int j = 0; j < RPT; ++j) s[j] *= e0;
        for (int ii = 0; ii < P.m; ++ii) {
            const f4 x = load4(vrs + ii * DV + c0);
            RawChunk<IO, RPT> krow;
            float kf[RPT];
            krow.load(krs + ii * DK + rg * RPT);
            krow.to_float(kf);
            const float w = fw[ii];
#pragma unroll
            for (int j = 0; j < RPT; ++j) s[j] += (w * kf[j]) * x;
        }
        float* wt = P.state + (static_cast<size_t>(slot) * P.H + h) * DK * DV;
#pragma unroll
        for (int j = 0; j < RPT; ++j)
            __builtin_nontemporal_store(s[j], reinterpret_cast<f4*>(wt + (rg * RPT + j) * DV + c0));
    }

    // ---- 8. metadata: occupancy over the appended tokens, table rotation -----
    if (tid < 64 && P.mode != MODE_VERIFY)  // drafts do not advance the occupancy
        update_meta(P, b, h, fold ? T - P.m : T, fold ? P.m / P.block_size : 0, tid, blk);
}

template <int RULE, int D, typename IO, bool TREE>
hipError_t launch_chunk_q(const TileParams& p, int batch, hipStream_t s) {
    using G = Geo<D, D>;
    const int cap = p.block_size * p.blocks_per_req;
    const int nq = p.n <= 1 ? 1 : p.n <= 2 ? 2 : p.n <= 4 ? 4 : 8;
    using XIO = typename std::conditional<RULE == KVBUF_RULE_DELTA, float, IO>::type;
    const size_t lds = sizeof(float) * chunk_lds(RULE, D, D, nq, G::RG, G::NT / 16, cap, p.m, p.fold_chunk > 0,
                                                 static_cast<int>(sizeof(IO)), static_cast<int>(sizeof(XIO))).total;
    const dim3 grid(static_cast<unsigned>(batch) * p.H), block(G::NT);
    switch (nq) {
        case 1: chunk_kernel<RULE, D, D, 1, IO, TREE><<<grid, block, lds, s>>>(p); break;
        case 2: chunk_kernel<RULE, D, D, 2, IO, TREE><<<grid, block, lds, s>>>(p); break;
        case 4: chunk_kernel<RULE, D, D, 4, IO, TREE><<<grid, block, lds, s>>>(p); break;
        default: chunk_kernel<RULE, D, D, 8, IO, TREE><<<grid, block, lds, s>>>(p); break;
    }
    return hipGetLastError();
}

template <int RULE, int D, typename IO>
hipError_t launch_chunk_t(const TileParams& p, int batch, hipStream_t s) {
    return p.parent ? launch_chunk_q<RULE, D, IO, true>(p, batch, s) : launch_chunk_q<RULE, D, IO, false>(p, batch, s);
}

template <int RULE, typename IO>
hipError_t launch_chunk_d(const TileParams& p, int d, int batch, hipStream_t s) {
    switch (d) {
        case 16: return launch_chunk_t<RULE, 16, IO>(p, batch, s);
        case 64: return launch_chunk_t<RULE, 64, IO>(p, batch, s);
        default: return launch_chunk_t<RULE, 128, IO>(p, batch, s);
    }
}

template <typename IO>
hipError_t launch_chunk_r(const TileParams& p, int rule, int d, int batch, hipStream_t s) {
    switch (rule) {
        case KVBUF_RULE_LINEAR: return launch_chunk_d<KVBUF_RULE_LINEAR, IO>(p, d, batch, s);
        case KVBUF_RULE_GATED: return launch_chunk_d<KVBUF_RULE_GATED, IO>(p, d, batch, s);
        default: return launch_chunk_d<KVBUF_RULE_DELTA, IO>(p, d, batch, s);
    }
}

}  // namespace

// The eager fold happens inside the decode launch when its m tokens fit what
// that kernel stages (the one-token kernel: an LDS budget; this kernel: the
// first staging pass of NT / 16 positions); otherwise a fold launch follows.
int chunk_fold_limit(int rule, int d, int io, int n, int cap, int m, int64_t tiles) {
    if (decode_eligible(rule, d, io, n, cap, m, tiles)) return decode_fold_limit(rule, d, io);
    if (rule == KVBUF_RULE_CHANNEL) return 0;  // the per-channel kernel never folds
    switch (d) {
        case 16: return Geo<16, 16>::NT / 16;
        case 64: return Geo<64, 64>::NT / 16;
        default: return Geo<128, 128>::NT / 16;
    }
}

hipError_t launch_chunk(const TileParams& p, int rule, int d, int io, int batch, hipStream_t s) {
    // (kvbuf_direct has a kernel of its own; requests without a state inside
    // a decode or verify launch are served here or by the one-token kernel.)
    if (!p.parent && decode_eligible(rule, d, io, p.n, p.block_size * p.blocks_per_req, p.m,
                                     static_cast<int64_t>(batch) * p.H))
        return launch_decode(p, rule, d, io, batch, s);
    if (rule == KVBUF_RULE_CHANNEL) return launch_channel(p, d, io, batch, s);
    return io == KVBUF_BF16 ? launch_chunk_r<bf16_bits>(p, rule, d, batch, s)
                            : launch_chunk_r<float>(p, rule, d, batch, s);
}

}  // namespace kvbuf
