// One-token decode for the linear and gated rules, with the work of a tile
// split between two roles that run at the same time.
//
// KVBuffer: IO-aware Serving for Linear Attention (pith.science page,
// Figure 1 caption: decode reads the state and the request's buffer blocks
// side by side; a full buffer is folded into the state, which goes back to
// its slot).  With b_i the cumulative
// log-gate since the last fold and t = p the new token's position:
//   o_t = e^{b_t} S0^T (scale q_t) + sum_{i<=t} e^{b_t - b_i} scale (q_t . k_i) v_i
//   fold (t = m - 1):  S <- e^{b_{m-1}} S0 + sum_{i<m} e^{b_{m-1} - b_i} k_i v_i^T
// With one log-gate per key channel (B_i the per-channel cumulative gate)
// every decay is a vector acting on the key channels:
//   o_t = S0^T (e^{B_t} scale q_t) + sum_{i<=t} scale (sum_r q_t[r] k_i[r] e^{B_t[r] - B_i[r]}) v_i
//   fold: row r of S0 scales by e^{B_{m-1}[r]}, k_i[r] by e^{B_{m-1}[r] - B_i[r]}.
//
// Serves kvbuf_decode and a one-draft kvbuf_verify when the table row covers
// at most 64 positions (one lane of the token wave per position), and
// kvbuf_direct of the per-channel rule (the other rules' buffer-only requests
// go to the chunk kernel).
//
// * State waves (NT threads): read the slot, issue the tile's 128-bit loads
//   at once (after only the query rows they multiply), and form their share
//   of S0^T q as soon as the tile arrives.  Nothing they issue depends on the
//   buffer metadata.
// * Token wave (64 lanes): occupancy and table row (one round trip), then the
//   keys, values and gates of every buffered position plus the new token (one
//   more), then scores, gate prefix sums, the weighted value sum, fold
//   staging and the appends -- all in registers and wave shuffles.
// The roles meet at one barrier; then the row-group partials are reduced into
// the output and, when the buffer fills, the state waves fold the staged
// tokens into the tile still held in registers and write it back.  The token
// wave, the tile's only reader of its occupancy and table row, advances them
// in place (decode, direct).
#include "device_common.hpp"

namespace kvbuf {
namespace {

__host__ __device__ inline int round4d(int x) { return (x + 3) & ~3; }

// LDS layout in 4-byte words.  mf = positions staged for a fold in this
// launch (0: it never folds); io = bytes per key / value element; for the
// per-channel rule, cap rows of gates (turned into per-channel suffix sums),
// the cumulative gate of the new token and the fold's per-row state decay;
// its fold keys are staged as fp32, already multiplied by their decays.
struct DecodeLds {
    int obuf, red, fw, kr, vr, dg, bt, qd, fr, ap, total;
};
__host__ __device__ inline DecodeLds decode_lds(int DK, int DV, int RG, int mf, int io, bool ch, int cap) {
    DecodeLds L;
    int o = 0;
    L.obuf = o; o += DV;                        // weighted sum of buffered values (token wave)
    L.red = o; o += RG * DV;                    // S0^T q partials, one row per row group
    L.fw = o; o += round4d(mf);                 // fold weights e^{b_{m-1} - b_i}
    L.kr = o; o += round4d(mf * DK * (ch ? 4 : io) / 4);  // keys to fold (raw bits; weighted fp32)
    L.vr = o; o += round4d(mf * DV * io / 4);   // values to fold (raw bits)
    L.dg = o; o += ch ? cap * DK : 0;           // per-channel rule: B_t - B_i per position (fp32)
    L.bt = o; o += ch ? DK : 0;                 // per-channel rule: e^{B_t}
    L.qd = o; o += ch ? DK : 0;                 // per-channel rule: e^{B_t} q_t
    L.fr = o; o += ch ? DK : 0;                 // per-channel rule: e^{B_{m-1} - B_t} per state row
    L.ap = o; o += round4d((DK + DV) * io / 4) + (ch ? DK : 0);  // the new token's key, value (, gate row)
    L.total = o;
    return L;
}

// bf16, d = 128, scalar or no gates: at most 80 registers, six waves per SIMD,
// so that a CU places four of these five-wave workgroups (each needs room for
// two of its waves on every SIMD) instead of three.
template <int RULE, int DK, int DV, typename IO>
__global__ __launch_bounds__((Geo<DK, DV>::NTHREADS))
__attribute__((amdgpu_waves_per_eu(DK == 128 && RULE != KVBUF_RULE_CHANNEL && sizeof(IO) == 2 ? 6 : 1)))
void decode_kernel(TileParams P) {
    using G = Geo<DK, DV>;
    constexpr int NT = G::NT, TPR = G::TPR, RG = G::RG, RPT = G::RPT;
    constexpr int E = DK / 16, EV = DV / 16;
    constexpr bool CH = RULE == KVBUF_RULE_CHANNEL;   // one gate per key channel
    // rounds of 4 positions whose loads are in flight together (the
    // per-channel rule's decayed dots need more registers per round)
    constexpr int NB = CH ? 2 : 4;
    constexpr bool GATED = RULE == KVBUF_RULE_GATED;  // one gate per token
    constexpr int CPL = (DK + 63) / 64;               // key channels per token-wave lane

    extern __shared__ __attribute__((aligned(16))) float lds[];  // 16-byte rows for the LDS copies
    __shared__ unsigned s_bad;
    __shared__ int s_fold;
    __shared__ float s_es, s_e0;
    // the token wave's stores, made after the barrier (see its end)
    __shared__ uint32_t s_arow;  // pool row of the new token
    __shared__ float s_ag;       // its log-gate (one per token)
    __shared__ int s_pnew, s_rot;
    __shared__ int s_blk[64];    // the table row as read

    const TileIndex ti = tile_index(P);
    const int b = ti.b;
    const int h = ti.h;
    const int tid = threadIdx.x;
    const bool token_wave = tid >= NT;
    const int rg = tid / TPR;
    const int c0 = (tid % TPR) * 4;
    const bool direct = P.mode == MODE_DIRECT;
    const int mf = P.fold_chunk;  // = m when this launch may fold
    const DecodeLds L = decode_lds(DK, DV, RG, mf, static_cast<int>(sizeof(IO)), CH,
                                   P.block_size * P.blocks_per_req);
    float* dg = lds + L.dg;
    float* btv = lds + L.bt;
    float* qdv = lds + L.qd;
    float* frow = lds + L.fr;
    float* krf = lds + L.kr;  // per-channel rule: weighted fp32 fold keys
    float* obuf = lds + L.obuf;
    float* red = lds + L.red;
    float* fw = lds + L.fw;
    IO* krs = reinterpret_cast<IO*>(lds + L.kr);
    IO* vrs = reinterpret_cast<IO*>(lds + L.vr);
    IO* kap = reinterpret_cast<IO*>(lds + L.ap);  // the new token's key, value and gate row
    IO* vap = kap + DK;
    float* gap = lds + L.ap + round4d((DK + DV) * static_cast<int>(sizeof(IO)) / 4);
    const size_t in_row = static_cast<size_t>(b) * P.H + h;  // one new token per request
    const int slot = direct ? -1 : P.slot[b];
    const IO* qin = static_cast<const IO*>(P.q) + in_row * DK;

    // ---- token wave ------------------------------------------------------------
    if (token_wave) {
        const int lane = tid - NT;
        const int bs = P.block_size;
        const int bpr = P.blocks_per_req;  // bs * bpr <= 64 (launcher)
        const int cap = bs * bpr;
        const int p = load_occupancy(P, b, h);
        int blk = 0;
        blk = load_table_row(P, b, h, lane);
        const int T = p + 1;  // positions after the append
        unsigned bad = 0;
        if (p < 0 || p >= cap) bad |= KVBUF_DEVERR_OVERFLOW;
        if (slot >= P.num_slots) bad |= KVBUF_DEVERR_SLOT;
        const int nblk = bad ? 0 : (T + bs - 1) / bs;
        if (__ballot(lane < nblk && (blk < 0 || blk >= P.num_blocks))) bad |= KVBUF_DEVERR_BLOCK;
        const int pc = bad ? 0 : p;  // p, clamped for the lane arithmetic below
        const bool fold = !bad && mf > 0 && slot >= 0 && T >= P.m;

        // pool row of position `lane` (host: num_blocks * H * block_size < 2^31)
        const int qb = min(lane / bs, 63);
        const uint32_t bi = static_cast<uint32_t>(__shfl(blk, qb, 64));
        const uint32_t prow = (bi * static_cast<uint32_t>(P.H) + static_cast<uint32_t>(h)) *
                                  static_cast<uint32_t>(bs) + static_cast<uint32_t>(lane - qb * bs);
        s_blk[lane] = blk;  // the table row as read, for the metadata update at the end

        const int gl = lane >> 4;  // position slot of the lane in a round
        const int cl = lane & 15;  // its 1/16 of a row
        const IO* kpool = static_cast<const IO*>(P.key);
        const IO* vpool = static_cast<const IO*>(P.value);
        const IO* kin = static_cast<const IO*>(P.k) + in_row * DK;
        const IO* vin = static_cast<const IO*>(P.v) + in_row * DV;
        const int Tl = bad ? 0 : T;

        // Issue every load of the first 4 * NB positions -- the gate of
        // position `lane`, the query chunk, keys and values -- before any is
        // used: one round trip after the table row.
        float g = 0.0f;
        if constexpr (GATED) {
            if (!bad && lane < pc) g = P.gate[prow];
            else if (!bad && lane == pc) g = P.g[in_row];
        }
        RawChunk<IO, E> qc;
        qc.load(qin + cl * E);
        // per-channel rule: this lane's channels of the query and of the new
        // token's gate row, loaded with the rest (each later use would
        // otherwise cost the chain a round trip); the query is kept as loaded
        // and widened where it is used (widening it here would wait for it,
        // and with it for every load above, before the rows are requested)
        IO qch[CH ? CPL : 1];
        float gnew[CH ? CPL : 1];
        if constexpr (CH) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int ch = lane + 64 * c;
                qch[c] = ch < DK ? qin[ch] : IO{};
                gnew[c] = ch < DK ? P.g[in_row * DK + ch] : 0.0f;
            }
        }
        RawChunk<IO, E> kc[NB];
        RawChunk<IO, EV> vc[NB];
        uint32_t pr[NB];
        auto issue = [&](int i0) {
#pragma unroll
            for (int r = 0; r < NB; ++r) {
                const int i = i0 + 4 * r + gl;
                pr[r] = static_cast<uint32_t>(__shfl(static_cast<int>(prow), i & 63, 64));
                kc[r].zero();
                vc[r].zero();
                if (i < pc) {
                    kc[r].load(kpool + static_cast<size_t>(pr[r]) * DK + cl * E);
                    vc[r].load(vpool + static_cast<size_t>(pr[r]) * DV + cl * EV);
                } else if (i == pc) {
                    kc[r].load(kin + cl * E);
                    vc[r].load(vin + cl * EV);
                }
            }
        };
        issue(0);
        if constexpr (CH) {
            // gate rows of every position straight into LDS, then in place
            // gate row i -> B_t - B_i (the gates after i up to t), per channel
            const float* gin = P.g + in_row * DK;
            lds_copy_rows<DK * 4>(reinterpret_cast<char*>(dg), Tl, [&](int i) {
                const uint32_t pri = static_cast<uint32_t>(__shfl(static_cast<int>(prow), i & 63, 64));
                return reinterpret_cast<const char*>(i < pc ? P.gate + static_cast<size_t>(pri) * DK : gin);
            }, lane);
            wait_lds_copies();
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int ch = lane + 64 * c;
                if (ch < DK) {
                    float run = 0.0f;
                    for (int i = Tl - 1; i >= 0; --i) {
                        const float gi = dg[i * DK + ch];
                        dg[i * DK + ch] = run;
                        run += gi;
                    }
                    const float ebt = exp_gate(run);
                    btv[ch] = ebt;                              // e^{B_t}
                    qdv[ch] = as_float(qch[c]) * ebt;           // e^{B_t} q
                    if (fold) frow[ch] = exp_gate(-dg[(P.m - 1) * DK + ch]);  // e^{B_{m-1} - B_t}
                }
            }
        }

        // cumulative log-gates b_i of positions 0 .. T-1, lane i holds b_i
        float bcum = 0.0f;
        if constexpr (GATED) {
            if (lane == pc) s_ag = g;  // the new token's log-gate, appended after the barrier
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(g, off, 64);
                if (lane >= off) g += y;
            }
            bcum = g;
        }
        const float bt = __shfl(bcum, pc, 64);

        float ob[EV];
#pragma unroll
        for (int e = 0; e < EV; ++e) ob[e] = 0.0f;
        for (int i0 = 0; i0 < Tl; i0 += 4 * NB) {
            if (i0 > 0) issue(i0);  // buffers longer than 4 * NB positions
#pragma unroll
            for (int r = 0; r < NB; ++r) {
                const int i = i0 + 4 * r + gl;
                float dot;
                if constexpr (CH) {
                    // sum_r q[r] (k_i[r] e^{B_t[r] - B_i[r]}); the decayed key is
                    // also the fold's key, up to the row factor e^{B_{m-1} - B_t}
                    float qf[E], kf[E], dd[E];
                    qc.to_float(qf);
                    kc[r].to_float(kf);
                    loadE<E>(dg + (i < Tl ? i : 0) * DK + cl * E, dd);
                    float acc = 0.f;
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        kf[e] *= exp_gate(dd[e]);
                        acc += qf[e] * kf[e];
                    }
                    dot = group16_sum(acc);
                    if (fold && i < P.m) {
#pragma unroll
                        for (int e = 0; e < E; ++e) krf[i * DK + cl * E + e] = kf[e];
                    }
                } else {
                    dot = group16_sum(chunk_dot(qc, kc[r]));
                }
                const float bi_ = __shfl(bcum, i & 63, 64);
                const float w = i < Tl ? (GATED ? exp_gate(bt - bi_) : 1.0f) * P.scale * dot : 0.0f;
                float vf[EV];
                vc[r].to_float(vf);
#pragma unroll
                for (int e = 0; e < EV; ++e) ob[e] += w * vf[e];
                if (fold && i < P.m) {
                    if constexpr (!CH) kc[r].store(krs + i * DK + cl * E);
                    vc[r].store(vrs + i * DV + cl * EV);
                }
                if (i == pc && i < Tl) {  // the new token, appended to the pool after the barrier
                    kc[r].store(kap + cl * E);
                    vc[r].store(vap + cl * EV);
                    if (cl == 0) s_arow = pr[r];
                }
            }
        }
        // sum the four position slots: lanes cl, cl+16, cl+32, cl+48
#pragma unroll
        for (int e = 0; e < EV; ++e) {
            ob[e] += __shfl_xor(ob[e], 16, 64);
            ob[e] += __shfl_xor(ob[e], 32, 64);
        }
        if (gl == 0) {
            // the columns from an opaque copy of the lane: formed here, not
            // kept in a register through the rounds
            int el = lane;
            asm volatile("" : "+v"(el));
#pragma unroll
            for (int e = 0; e < EV; ++e) obuf[(el & 15) * EV + e] = ob[e];
        }
        if constexpr (CH) {  // the new token's gate row
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int ch = lane + 64 * c;
                if (ch < DK) gap[ch] = gnew[c];
            }
        }
        if (fold && !CH) {
            const float bm = __shfl(bcum, P.m - 1, 64);
            if (lane < P.m) fw[lane] = GATED ? exp_gate(bm - bcum) : 1.0f;
            if (lane == 0) s_e0 = GATED ? exp_gate(bm) : 1.0f;
        }
        if (lane == 0) {
            s_bad = bad;
            s_fold = fold ? 1 : 0;
            s_es = GATED ? exp_gate(bt) : 1.0f;
        }
        // this wave read the tile's metadata above; it advances it in place
        // after the barrier (the table row is in s_blk)
        if (lane == 0) {
            s_pnew = fold ? Tl - P.m : Tl;
            s_rot = fold ? P.m / bs : 0;
        }
    }

    // ---- state waves: query rows, then the tile; S0^T q per row group ----------
    f4 s[RPT];
    RawChunk<IO, RPT> qrow;
    if (!token_wave) {
        if constexpr (!CH) qrow.load(qin + rg * RPT);
        const bool present = slot >= 0 && slot < P.num_slots;
        load_tile<RPT, DK, DV>(s, present ? P.state + (static_cast<size_t>(slot) * P.H + h) * DK * DV : P.state,
                               present, rg, c0);
        if constexpr (!CH) {
            f4 sa = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < RPT; ++j) sa += s[j] * qrow.at(j);
            *reinterpret_cast<f4*>(red + rg * DV + c0) = sa;
        }
    }
    if constexpr (CH) {
        // S0^T (e^{B_t} q) needs the token wave's B_t: one more barrier
        __syncthreads();
        if (!token_wave) {
            float qf[RPT];
            loadE<RPT>(qdv + rg * RPT, qf);
            f4 sa = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < RPT; ++j) sa += s[j] * qf[j];
            *reinterpret_cast<f4*>(red + rg * DV + c0) = sa;
        }
    }
    __syncthreads();
    if (s_bad) {
        report(P, s_bad);
        return;  // the tile is skipped and its metadata left unchanged
    }

    // ---- token wave: its stores, after the barrier (which would wait for
    // them): the new token's key, value and gate, and the metadata ----------------
    if (token_wave) {
        const int lane = tid - NT;
        const size_t row = s_arow;
        if (lane < 16) {
            RawChunk<IO, E> kc;
            kc.load(kap + lane * E);
            kc.store(static_cast<IO*>(P.key) + row * DK + lane * E);
        } else if (lane < 32) {
            RawChunk<IO, EV> vc;
            vc.load(vap + (lane - 16) * EV);
            vc.store(static_cast<IO*>(P.value) + row * DV + (lane - 16) * EV);
        }
        if constexpr (GATED) {
            if (lane == 0) P.gate[row] = s_ag;
        }
        if constexpr (CH) {
            for (int ch = lane; ch < DK; ch += 64) P.gate[row * DK + ch] = gap[ch];
        }
        if (P.mode != MODE_VERIFY) update_meta(P, b, h, s_pnew, s_rot, lane, s_blk[lane]);
        return;
    }

    // ---- output: e^{b_t} scale (S0^T q) + buffered part ---------------------------
    if (tid < DV) {
        float sum = 0.f;
#pragma unroll
        for (int g2 = 0; g2 < RG; ++g2) sum += red[g2 * DV + tid];
        store_out(P, in_row * DV + tid, sum * (CH ? P.scale : P.scale * s_es) + obuf[tid]);
    }

    // ---- eager fold: the buffer reached m tokens ---------------------------------
    if (s_fold && !token_wave) {
        if constexpr (CH) {
            // e^{B_{m-1} - B_t} (e^{B_t} S0 + sum_i k_i e^{B_t - B_i} v_i^T), row by
            // row; the staged keys carry their decays e^{B_t - B_i}
#pragma unroll
            for (int j = 0; j < RPT; ++j) s[j] *= btv[rg * RPT + j];
            for (int ii = 0; ii < P.m; ++ii) {
                const f4 x = load4(vrs + ii * DV + c0);
                float kf[RPT];
                loadE<RPT>(krf + ii * DK + rg * RPT, kf);
#pragma unroll
                for (int j = 0; j < RPT; ++j) s[j] += kf[j] * x;
            }
#pragma unroll
            for (int j = 0; j < RPT; ++j) s[j] *= frow[rg * RPT + j];
        } else {
            const float e0 = s_e0;
#pragma unroll
            for (int j = 0; j < RPT; ++j) s[j] *= e0;
            for (int ii = 0; ii < P.m; ++ii) {
                // the weight goes with the value (4 products, not 16); the
                // keys are widened one at a time as they are used
                const f4 wx = fw[ii] * load4(vrs + ii * DV + c0);
                RawChunk<IO, RPT> krow;
                krow.load(krs + ii * DK + rg * RPT);
#pragma unroll
                for (int j = 0; j < RPT; ++j) s[j] += krow.at(j) * wx;
            }
        }
        float* wt = P.state + (static_cast<size_t>(slot) * P.H + h) * DK * DV;
        // the thread's rows and columns from an opaque copy of its index:
        // formed here, not kept in registers through the kernel
        int et = tid;
        asm volatile("" : "+v"(et));
        const int rgs = et / TPR, cs = (et % TPR) * 4;
#pragma unroll
        for (int j = 0; j < RPT; ++j)
            __builtin_nontemporal_store(s[j], reinterpret_cast<f4*>(wt + (rgs * RPT + j) * DV + cs));
    }
}

template <int RULE, int D, typename IO>
hipError_t launch_decode_t(const TileParams& p, int batch, hipStream_t s) {
    using G = Geo<D, D>;
    const size_t lds = sizeof(float) * decode_lds(D, D, G::RG, p.fold_chunk, static_cast<int>(sizeof(IO)),
                                                  RULE == KVBUF_RULE_CHANNEL, p.block_size * p.blocks_per_req).total;
    decode_kernel<RULE, D, D, IO><<<dim3(static_cast<unsigned>(batch) * p.H), dim3(G::NTHREADS), lds, s>>>(p);
    return hipGetLastError();
}

template <int RULE, typename IO>
hipError_t launch_decode_d(const TileParams& p, int d, int batch, hipStream_t s) {
    switch (d) {
        case 16: return launch_decode_t<RULE, 16, IO>(p, batch, s);
        case 64: return launch_decode_t<RULE, 64, IO>(p, batch, s);
        default: return launch_decode_t<RULE, 128, IO>(p, batch, s);
    }
}

}  // namespace

// Largest m a decode launch of this kernel folds itself: the keys and values
// of the m positions are staged in LDS (at most 32 KiB of them; fp32 keys for
// the per-channel rule).
int decode_fold_limit(int rule, int d, int io) {
    const int e = io == KVBUF_BF16 ? 2 : 4;
    const int bytes_per_pos = d * e + d * (rule == KVBUF_RULE_CHANNEL ? 4 : e);
    return 32768 / bytes_per_pos;
}

bool decode_eligible(int rule, int d, int io, int n, int cap, int m, int64_t tiles) {
    if (rule == KVBUF_RULE_DELTA || n != 1 || cap > 64) return false;
    if (rule == KVBUF_RULE_CHANNEL) return true;
    // A launch of a few workgroup generations (d = 128, bf16) goes to the
    // chunk kernel when it folds there too (m within its first staging pass).
    // Both kernels hold four tiles per CU; at these sizes the last, partial
    // generation decides, and the chunk kernel's is as short or shorter.
    // Measured, B * H = 1024 / 2048 tiles: 0.698 / 0.695 of the HBM peak
    // against 0.700 / 0.689 here.
    const bool few = d == 128 && io == KVBUF_BF16 && tiles <= kFewTiles && m <= Geo<128, 128>::NT / 16;
    return !few;
}

hipError_t launch_decode(const TileParams& p, int rule, int d, int io, int batch, hipStream_t s) {
    if (rule == KVBUF_RULE_CHANNEL)
        return io == KVBUF_BF16 ? launch_decode_d<KVBUF_RULE_CHANNEL, bf16_bits>(p, d, batch, s)
                                : launch_decode_d<KVBUF_RULE_CHANNEL, float>(p, d, batch, s);
    if (rule == KVBUF_RULE_LINEAR)
        return io == KVBUF_BF16 ? launch_decode_d<KVBUF_RULE_LINEAR, bf16_bits>(p, d, batch, s)
                                : launch_decode_d<KVBUF_RULE_LINEAR, float>(p, d, batch, s);
    return io == KVBUF_BF16 ? launch_decode_d<KVBUF_RULE_GATED, bf16_bits>(p, d, batch, s)
                            : launch_decode_d<KVBUF_RULE_GATED, float>(p, d, batch, s);
}

}  // namespace kvbuf
