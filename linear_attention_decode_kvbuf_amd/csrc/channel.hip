// Decode and draft verification under the per-channel decay rule (one
// log-gate per key channel) for the cases the one-token kernel does not
// serve: several drafts (a chain or a tree) and table rows of more than 64
// positions.
//
// KVBuffer: IO-aware Serving for Linear Attention (pith.science page; its
// reference list includes gated linear attention and matrix-state RNNs,
// whose decays act per key channel).  With g_s the gate row of position s
// and the buffer holding positions 0 .. p-1, draft d (position p + d) gives
//   o_d = S0^T (e^{B_{p+d}} o q_d) + sum_{i seen by d} scale (sum_c q_d[c] k_i[c] e^{B_{p+d}[c] - B_i[c]}) v_i
// (o = per-channel product, B the cumulative gate row from position 0;
// "seen": the buffer, and the drafts on d's path, d included).  Every decay
// is split at the last buffered position p - 1:
//   R_i  = sum_{s=i+1}^{p-1} g_s   (buffered i; the gates after it in the buffer)
//   D_d  = sum of g over d's path of drafts (d included)
//   e^{B_{p+d} - B_i} = e^{D_d} e^{R_i}            (i < p)
//                     = e^{D_d} e^{-D_e}           (i = p + e, e on d's path)
//   e^{B_{p+d}}       = e^{D_d} e^{B_{p-1}}
// so with q^_d = scale q_d o e^{D_d}, every score is a plain dot product of
// q^_d with k_i o e^{R_i} (buffer) or k_{p+e} o e^{-D_e} (drafts), and the
// state query is q^_d o e^{B_{p-1}}.  R_i and B_{p-1} are sums of decays
// (at most 1 after exponentiation for log-gates <= 0) and D is a sum over at
// most 8 drafts, so no factor grows large.
//
// One workgroup per (request, head), NT threads holding the state tile (as
// the chunk kernel).  The buffered positions are visited newest first in
// passes of NT / 16: the key, value and gate rows of a pass are copied
// straight into a two-slot LDS ring; the threads that own a key channel walk
// the pass's positions from the newest back, turning its gate rows in place
// into the factors e^{R_i} while carrying R in a register; the scores and the
// weighted value sums follow.  The next pass is in flight meanwhile (the
// barriers between passes do not wait for copies; each wave counts its own).
// A decode that fills the buffer under the eager policy is folded by the
// launch that follows (the fold kernel).
#include "device_common.hpp"

namespace kvbuf {
namespace {

// LDS layout in 4-byte words (launcher and kernel).
struct ChannelLds {
    int pos, cq, qh, fd, gd, er, kd, vd, ring, total;
};

__host__ __device__ inline int r4c(int x) { return (x + 3) & ~3; }

__host__ __device__ inline ChannelLds channel_lds(int DK, int DV, int NQ, int RG, int NG, int cap, int io) {
    ChannelLds L;
    int o = 0;
    L.pos = o; o += r4c(cap);                 // pool row of each buffer position
    L.cq = o; o += NQ * r4c(cap + NQ);        // scores of each query against every position
    L.qh = o; o += NQ * DK;                   // scale q_d e^{D_d}
    L.fd = o; o += NQ * DK;                   // e^{-D_e} of each draft
    L.gd = o; o += NQ * DK;                   // the drafts' gate rows (appended at the end)
    L.er = o; o += DK;                        // e^{B_{p-1}}
    L.kd = o; o += r4c(NQ * DK * io / 4);     // the drafts' keys (raw)
    L.vd = o; o += r4c(NQ * DV * io / 4);     // their values (raw)
    L.ring = o;                               // two passes of key, value and gate rows;
    const int ring = 2 * NG * (DK * io + DV * io + DK * 4) / 4;  // then the row-group partials
    const int red = RG * DV * NQ;
    o += ring > red ? ring : red;
    L.total = o;
    return L;
}

// The barrier between the phases of a pass: LDS accesses complete, copies
// still in flight stay in flight (each wave waits for its own copies first).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int DK, int DV, int NQ, typename IO, bool TREE>
__global__ __launch_bounds__((Geo<DK, DV>::NT)) void channel_kernel(TileParams P) {
    using G = Geo<DK, DV>;
    constexpr int NT = G::NT, TPR = G::TPR, RG = G::RG, RPT = G::RPT;
    constexpr int E = DK / 16;
    constexpr int NG = NT / 16;               // positions per pass
    constexpr int NQR = (NQ + NG - 1) / NG;   // draft rows per thread
    constexpr int IOB = static_cast<int>(sizeof(IO));
    constexpr int KB = DK * IOB, VB = DV * IOB, GB = DK * 4;  // row bytes
    constexpr int RW = NG / (NT / 64);        // rows of a pass each wave copies
    static_assert(RW == 4 && NT >= DK, "pass geometry");
    // copy instructions of one full pass per wave (lds_copy_rows: 1 KiB each)
    constexpr int FULL = (RW + 64 / (KB / 16) - 1) / (64 / (KB / 16)) + (RW + 64 / (VB / 16) - 1) / (64 / (VB / 16)) +
                         (RW + 64 / (GB / 16) - 1) / (64 / (GB / 16));
    static_assert(FULL < 16, "vmcnt low field");

    extern __shared__ __attribute__((aligned(16))) float lds[];
    __shared__ unsigned s_bad;
    __shared__ int s_p;
    __shared__ uint32_t s_anc[TREE ? kMaxDrafts : 1];

    const TileIndex ti = tile_index(P);
    const int b = ti.b, h = ti.h;
    const int tid = threadIdx.x;
    const int rg = tid / TPR, c0 = (tid % TPR) * 4;
    const int gp = tid >> 4, cl = tid & 15;
    const int n = P.n;
    const int cap = P.block_size * P.blocks_per_req;
    const ChannelLds L = channel_lds(DK, DV, NQ, RG, NG, cap, IOB);
    uint32_t* spos = reinterpret_cast<uint32_t*>(lds + L.pos);
    float* cq = lds + L.cq;
    const int ldc = r4c(cap + NQ);
    float* qh = lds + L.qh;
    float* fd = lds + L.fd;
    float* gd = lds + L.gd;
    float* er = lds + L.er;
    IO* kd = reinterpret_cast<IO*>(lds + L.kd);
    IO* vd = reinterpret_cast<IO*>(lds + L.vd);
    char* ring = reinterpret_cast<char*>(lds + L.ring);
    constexpr int SLOT = NG * (KB + VB + GB);  // bytes of one ring slot: keys, values, gates
    float* red = lds + L.ring;                 // after the last pass

    // ---- metadata (wave 0), then the state tile -----------------------------------
    const int slot = P.slot[b];
    int p0 = 0, blk = 0, par = -1;
    if (tid < 64) {
        p0 = load_occupancy(P, b, h);
        blk = load_table_row(P, b, h, tid);
        if (TREE && tid < n) par = P.parent[static_cast<size_t>(b) * n + tid];
    }
    f4 s[RPT];
    __builtin_amdgcn_sched_barrier(0);
    {
        const bool present = slot >= 0 && slot < P.num_slots;
        load_tile<RPT, DK, DV>(s, present ? P.state + (static_cast<size_t>(slot) * P.H + h) * DK * DV : P.state,
                               present, rg, c0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (tid < 64) {
        unsigned bad = stage_row_from(P, h, (p0 < 0 || p0 > cap) ? -1 : p0 + n, spos, tid, blk);
        if (slot >= P.num_slots) bad |= KVBUF_DEVERR_SLOT;
        if constexpr (TREE) {
            const bool bad_par = tid < n && (par < -1 || par >= tid);  // parents precede children
            if (__ballot(bad_par)) bad |= KVBUF_DEVERR_ACCEPT;
            uint32_t anc = 0;  // draft tid and its ancestors
            int cur = (tid < n && !bad_par) ? tid : -1;
            for (int step = 0; step < n; ++step) {
                if (cur >= 0) anc |= 1u << cur;
                const int up = __shfl(par, cur >= 0 ? cur : 0, 64);
                cur = (cur > 0 && up >= 0 && up < cur) ? up : -1;
            }
            if (tid < n) s_anc[tid] = anc;
        }
        if (tid == 0) {
            s_bad = bad;
            s_p = p0;
        }
    }
    __syncthreads();
    if (s_bad) {
        report(P, s_bad);
        return;  // the tile is skipped and its metadata left unchanged
    }
    const int p = s_p;
    const bool has_state = slot >= 0;
    const size_t in_row = static_cast<size_t>(b) * n * P.H + h;  // (b, draft 0, h)
    const size_t in_stride = static_cast<size_t>(P.H);          // draft d at in_row + d * H
    auto seen = [&](int d, int e) { return TREE ? ((s_anc[TREE ? d : 0] >> e) & 1u) != 0 : e <= d; };

    // ---- the drafts: keys and values to LDS; channel owners: gates, D, q^ ---------
    RawChunk<IO, E> kdr[NQR], vdr[NQR];
#pragma unroll
    for (int r = 0; r < NQR; ++r) {
        const int d = gp + NG * r;
        kdr[r].zero();
        vdr[r].zero();
        if (d < n) {
            kdr[r].load(static_cast<const IO*>(P.k) + (in_row + d * in_stride) * DK + cl * E);
            vdr[r].load(static_cast<const IO*>(P.v) + (in_row + d * in_stride) * DV + cl * (DV / 16));
        }
    }
    // channel owners: the drafts' gates and queries of channel tid (the
    // queries kept as loaded and widened where used: widening them here would
    // wait for them, and with them for the state tile requested above)
    float gdr[NQ];
    IO qv[NQ];
#pragma unroll
    for (int d = 0; d < NQ; ++d) {
        gdr[d] = 0.f;
        qv[d] = IO{};
        if (tid < DK && d < n) {
            gdr[d] = P.g[(in_row + d * in_stride) * DK + tid];
            qv[d] = static_cast<const IO*>(P.q)[(in_row + d * in_stride) * DK + tid];
        }
    }

    // ---- the two newest passes of buffered rows, copied straight to the ring ------
    const int npass = (p + NG - 1) / NG;
    auto pass_base = [&](int r) { return (npass - 1 - r) * NG; };  // newest first
    auto copy_pass = [&](int r) {
        const int i0 = pass_base(r);
        char* base = ring + (r & 1) * SLOT;
        const int w = tid >> 6, lane = tid & 63;
        const int r0 = w * RW;
        const int cnt = max(0, min(RW, p - (i0 + r0)));
        auto row = [&](int k) -> size_t { return spos[i0 + r0 + k]; };
        lds_copy_rows<KB>(base + r0 * KB, cnt,
                          [&](int k) { return reinterpret_cast<const char*>(static_cast<const IO*>(P.key) + row(k) * DK); },
                          lane);
        lds_copy_rows<VB>(base + NG * KB + r0 * VB, cnt,
                          [&](int k) { return reinterpret_cast<const char*>(static_cast<const IO*>(P.value) + row(k) * DV); },
                          lane);
        lds_copy_rows<GB>(base + NG * (KB + VB) + r0 * GB, cnt,
                          [&](int k) { return reinterpret_cast<const char*>(P.gate + row(k) * DK); }, lane);
    };
    if (npass > 0) copy_pass(0);
    if (npass > 1) copy_pass(1);
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int r = 0; r < NQR; ++r) {
        const int d = gp + NG * r;
        if (d < n) {
            kdr[r].store(kd + d * DK + cl * E);
            vdr[r].store(vd + d * DV + cl * (DV / 16));
        }
    }
    if (tid < DK) {
#pragma unroll
        for (int d = 0; d < NQ; ++d) {
            float D = 0.f;  // the gates of d's path, in draft order
#pragma unroll
            for (int e = 0; e < NQ; ++e)
                if (e < n && d < n && seen(d, e)) D += gdr[e];
            if (d < n) {
                qh[d * DK + tid] = P.scale * as_float(qv[d]) * exp_gate(D);
                fd[d * DK + tid] = exp_gate(-D);
                gd[d * DK + tid] = gdr[d];
            }
        }
    }

    // ---- buffered passes, newest first -----------------------------------------------
    f4 acc[NQ];
#pragma unroll
    for (int d = 0; d < NQ; ++d) acc[d] = f4{0.f, 0.f, 0.f, 0.f};
    float R = 0.f;  // channel owners: sum of the gates after the position visited
    for (int r = 0; r < npass; ++r) {
        // this wave's copies of pass r have landed (pass r + 1, if any, may be in flight)
        if (r + 1 < npass) __builtin_amdgcn_s_waitcnt((FULL & 15) | 0x0F70);
        else __builtin_amdgcn_s_waitcnt(0x0F70);
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        const int i0 = pass_base(r);
        const int cnt = min(NG, p - i0);
        const char* base = ring + (r & 1) * SLOT;
        float* gf = reinterpret_cast<float*>(const_cast<char*>(base) + NG * (KB + VB));
        if (tid < DK) {
            for (int k = cnt - 1; k >= 0; --k) {
                const float gk = gf[k * DK + tid];
                gf[k * DK + tid] = exp_gate(R);  // e^{R_i}
                R += gk;
            }
        }
        lds_barrier();
        // scores: thread (gp, cl) against position i0 + gp
        if (gp < cnt) {
            RawChunk<IO, E> kc;
            kc.load(reinterpret_cast<const IO*>(base) + gp * DK + cl * E);
            float kf[E], ff[E];
            kc.to_float(kf);
            loadE<E>(gf + gp * DK + cl * E, ff);
#pragma unroll
            for (int e = 0; e < E; ++e) kf[e] *= ff[e];
#pragma unroll
            for (int d = 0; d < NQ; ++d) {
                if (d < n) {
                    float qf[E];
                    loadE<E>(qh + d * DK + cl * E, qf);
                    float dot = 0.f;
#pragma unroll
                    for (int e = 0; e < E; ++e) dot += qf[e] * kf[e];
                    dot = group16_sum(dot);
                    if (cl == 0) cq[d * ldc + i0 + gp] = dot;
                }
            }
        }
        lds_barrier();
        // weighted sums: row group rg takes the pass positions rg, rg + RG, ...
        const IO* vb = reinterpret_cast<const IO*>(base + NG * KB);
        for (int ii = rg; ii < cnt; ii += RG) {
            const f4 x = load4(vb + ii * DV + c0);
#pragma unroll
            for (int d = 0; d < NQ; ++d)
                if (d < n) acc[d] += cq[d * ldc + i0 + ii] * x;
        }
        if (r + 2 < npass) {
            lds_barrier();  // every wave is done with this slot
            copy_pass(r + 2);
        }
    }
    if (tid < DK) er[tid] = exp_gate(R);  // e^{B_{p-1}}
    __syncthreads();  // q^ and e^{-D} (an empty buffer has had no barrier since)

    // ---- the drafts' positions ----------------------------------------------------
#pragma unroll
    for (int r = 0; r < NQR; ++r) {
        const int e = gp + NG * r;  // draft e at position p + e
        if (e < n) {
            RawChunk<IO, E> kc;
            kc.load(kd + e * DK + cl * E);
            float kf[E], ff[E];
            kc.to_float(kf);
            loadE<E>(fd + e * DK + cl * E, ff);
#pragma unroll
            for (int c = 0; c < E; ++c) kf[c] *= ff[c];
#pragma unroll
            for (int d = 0; d < NQ; ++d) {
                if (d < n) {
                    float qf[E];
                    loadE<E>(qh + d * DK + cl * E, qf);
                    float dot = 0.f;
#pragma unroll
                    for (int c = 0; c < E; ++c) dot += qf[c] * kf[c];
                    dot = group16_sum(dot);
                    if (cl == 0) cq[d * ldc + p + e] = seen(d, e) ? dot : 0.f;
                }
            }
        }
    }
    __syncthreads();
    for (int e = rg; e < n; e += RG) {
        const f4 x = load4(vd + e * DV + c0);
#pragma unroll
        for (int d = 0; d < NQ; ++d)
            if (d < n) acc[d] += cq[d * ldc + p + e] * x;
    }

    // ---- the state: S0^T (q^_d o e^{B_{p-1}}), reduced with the buffer sums ----------
#pragma unroll
    for (int d = 0; d < NQ; ++d) {
        if (d < n) {
            f4 a = acc[d];
            if (has_state) {
                float qf[RPT], ef[RPT];
                loadE<RPT>(qh + d * DK + rg * RPT, qf);
                loadE<RPT>(er + rg * RPT, ef);
                f4 sa = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < RPT; ++j) sa += s[j] * (qf[j] * ef[j]);
                a += sa;
            }
            *reinterpret_cast<f4*>(red + (d * RG + rg) * DV + c0) = a;
        }
    }
    __syncthreads();
    const size_t outp = in_row * DV;  // output element of (request, draft 0, head)
    for (int idx = tid; idx < n * DV; idx += NT) {
        const int d = idx / DV;
        const int c = idx - d * DV;
        float sum = 0.f;
#pragma unroll
        for (int g2 = 0; g2 < RG; ++g2) sum += red[(d * RG + g2) * DV + c];
        store_out(P, outp + d * in_stride * DV + c, sum);
    }

    // ---- appends: the drafts' key, value and gate rows; metadata (decode) ------------
#pragma unroll
    for (int r = 0; r < NQR; ++r) {
        const int d = gp + NG * r;
        if (d < n) {
            const size_t row = spos[p + d];
            kdr[r].store(static_cast<IO*>(P.key) + row * DK + cl * E);
            vdr[r].store(static_cast<IO*>(P.value) + row * DV + cl * (DV / 16));
        }
    }
    if (tid < DK) {
#pragma unroll
        for (int d = 0; d < NQ; ++d)
            if (d < n) P.gate[static_cast<size_t>(spos[p + d]) * DK + tid] = gd[d * DK + tid];
    }
    if (tid < 64 && P.mode == MODE_DECODE) update_meta(P, b, h, p + n, 0, tid, blk);
}

template <int D, typename IO, bool TREE>
hipError_t launch_channel_t(const TileParams& p, int batch, hipStream_t s) {
    using G = Geo<D, D>;
    const int cap = p.block_size * p.blocks_per_req;
    const int nq = p.n <= 1 ? 1 : p.n <= 2 ? 2 : p.n <= 4 ? 4 : 8;
    const size_t lds = sizeof(float) * channel_lds(D, D, nq, G::RG, G::NT / 16, cap, static_cast<int>(sizeof(IO))).total;
    const dim3 grid(static_cast<unsigned>(batch) * p.H), block(G::NT);
    switch (nq) {
        case 1: channel_kernel<D, D, 1, IO, TREE><<<grid, block, lds, s>>>(p); break;
        case 2: channel_kernel<D, D, 2, IO, TREE><<<grid, block, lds, s>>>(p); break;
        case 4: channel_kernel<D, D, 4, IO, TREE><<<grid, block, lds, s>>>(p); break;
        default: channel_kernel<D, D, 8, IO, TREE><<<grid, block, lds, s>>>(p); break;
    }
    return hipGetLastError();
}

template <typename IO>
hipError_t launch_channel_d(const TileParams& p, int d, int batch, hipStream_t s) {
    const bool tree = p.parent != nullptr;
    switch (d) {
        case 16: return tree ? launch_channel_t<16, IO, true>(p, batch, s) : launch_channel_t<16, IO, false>(p, batch, s);
        case 64: return tree ? launch_channel_t<64, IO, true>(p, batch, s) : launch_channel_t<64, IO, false>(p, batch, s);
        default:
            return tree ? launch_channel_t<128, IO, true>(p, batch, s) : launch_channel_t<128, IO, false>(p, batch, s);
    }
}

}  // namespace

hipError_t launch_channel(const TileParams& p, int d, int io, int batch, hipStream_t s) {
    return io == KVBUF_BF16 ? launch_channel_d<bf16_bits>(p, d, batch, s) : launch_channel_d<float>(p, d, batch, s);
}

}  // namespace kvbuf
