// Buffered decode, draft verification and buffer-only decode (one kernel).
//
// KVBuffer: IO-aware Serving for Linear Attention (pith.science page):
//  * Figure 1 caption -- the output of a token is computed from the state,
//    loaded together with the buffered keys and values; once the buffer holds
//    m tokens the state is updated with all of them and written back;
//  * Figure 2 caption -- draft tokens are buffered and verified together,
//    without a temporary state per draft;
//  * abstract -- short contexts are served from the buffered keys and values
//    alone, without creating or updating a state.
//
// Unrolling the recurrence from the state S0 at the last fold (positions
// 0 .. T-1 buffered since then, b_i = g_0 + ... + g_i the cumulative log-gate):
//   o_t = e^{b_t} S0^T q_t + sum_{i<=t} e^{b_t - b_i} (q_t . k_i) x_i
//   S_t = e^{b_t} S0 + sum_{i<=t} e^{b_t - b_i} k_i x_i^T
// with x_i = v_i for the linear (b = 0) and gated rules, and for the delta rule
//   x_t = u_t = beta_t (v_t - e^{b_t} S0^T k_t - sum_{i<t} e^{b_t - b_i} (k_i . k_t) u_i),
// the pseudo-value the pool stores in place of v.
//
// One workgroup per (request, head).  The state waves issue all loads of the
// 64 KiB state tile (128-bit, non-temporal: the tile is not reused before it
// is evicted) and wait at a barrier; meanwhile the token wave forms the gate
// prefix sums, the q . k scores and the decay-weighted sum of the buffered
// values, and appends the new tokens to the pool.  After the barrier the state
// waves reduce S^T q from registers.  The state is the only large operand, so
// the kernel is bound by HBM bandwidth.
#include "device_common.hpp"

namespace kvbuf {
namespace {

// LDS layout of the chunk kernel, in floats.  Shared by the launcher (size)
// and the kernel (offsets).
struct ChunkLds {
    int qs, ks, bl, cq, ck, es, bq, bk, sq, sk, un, red, fk, fx, fw, total;
};

__host__ __device__ inline int round4(int x) { return (x + 3) & ~3; }

__host__ __device__ inline ChunkLds chunk_lds(int rule, int DK, int DV, int NQ, int RG, int cap, int fold_chunk) {
    ChunkLds L;
    int o = 0;
    const bool delta = rule == KVBUF_RULE_DELTA;
    L.qs = o; o += NQ * DK;                       // scaled queries of the new tokens
    L.ks = o; o += delta ? NQ * DK : 0;           // keys of the new tokens (delta rule)
    L.bl = o; o += round4(cap);                   // cumulative log-gates
    L.cq = o; o += NQ * round4(cap);              // e^{b_t - b_i} (q_t . k_i)
    L.ck = o; o += delta ? NQ * round4(cap) : 0;  // e^{b_t - b_i} (k_t . k_i)
    L.es = o; o += round4(NQ + 1);                // e^{b_t} per draft; [NQ]: e^{b_{m-1}}
    L.bq = o; o += NQ * DV;                       // sum_i cq_i x_i (buffered values)
    L.bk = o; o += delta ? NQ * DV : 0;           // sum_i ck_i x_i
    L.sq = o; o += delta ? NQ * DV : 0;           // reduced e^{b_t} S0^T q_t + bq
    L.sk = o; o += delta ? NQ * DV : 0;           // reduced e^{b_t} S0^T k_t + bk
    L.un = o; o += delta ? NQ * DV : 0;           // pseudo-values of the new tokens
    L.red = o; o += RG * DV * (delta ? 2 : 1);    // row-group partial sums
    L.fk = o; o += fold_chunk * DK;               // fold staging: keys,
    L.fx = o; o += fold_chunk * DV;               //   values,
    L.fw = o; o += round4(fold_chunk);            //   weights
    L.total = o;
    return L;
}

template <int RULE, int DK, int DV, int NQ, typename IO>
__global__ __launch_bounds__((Geo<DK, DV>::NTHREADS)) void chunk_kernel(TileParams P) {
    using G = Geo<DK, DV>;
    constexpr int NT = G::NT, TPR = G::TPR, RG = G::RG, RPT = G::RPT, CPL = G::CPL;
    constexpr bool DELTA = RULE == KVBUF_RULE_DELTA;
    constexpr bool GATED = RULE != KVBUF_RULE_LINEAR;
    using XIO = typename std::conditional<DELTA, float, IO>::type;

    extern __shared__ float lds[];
    __shared__ int32_t s_row[kMaxTableRow];
    __shared__ int s_last;

    const int tile = blockIdx.x;
    const int b = tile / P.H;
    const int h = tile - b * P.H;
    const int tid = threadIdx.x;
    const bool token_wave = tid >= NT;
    const int lane = tid - NT;  // token-wave lane
    const int rg = tid / TPR;
    const int c0 = (tid % TPR) * 4;
    const int n = P.n;
    const int cap = P.block_size * P.blocks_per_req;
    const bool direct = P.mode == MODE_DIRECT;

    const int p = P.occ[b];
    const int slot = direct ? -1 : P.slot[b];
    unsigned bad = (p < 0) ? KVBUF_DEVERR_OVERFLOW : load_row(P, b, p + n, s_row, NT);
    if (slot >= P.num_slots) bad |= KVBUF_DEVERR_SLOT;
    if (bad) {
        report(P, bad);
        return;  // the whole request is skipped by all of its workgroups
    }
    const bool has_state = slot >= 0;
    const int T = p + n;  // positions touched by this call
    const int fc = P.fold_chunk;  // > 0 only when this launch may fold (then fc >= m)
    const bool fold = fc > 0 && has_state && T >= P.m;

    const ChunkLds L = chunk_lds(RULE, DK, DV, NQ, RG, cap, fc);
    float* qs = lds + L.qs;
    float* ks = lds + L.ks;
    float* bl = lds + L.bl;
    float* cq = lds + L.cq;
    float* ck = lds + L.ck;
    float* es = lds + L.es;
    float* fk = lds + L.fk;
    float* fx = lds + L.fx;
    float* fw = lds + L.fw;
    const int ldc = round4(cap);

    const size_t in_row = static_cast<size_t>(b) * n * P.H + h;  // (b, draft 0, h)
    TileTokens<DK, DV, IO, XIO> tok;
    tok.kpool = static_cast<const IO*>(P.key);
    tok.xpool = static_cast<const XIO*>(P.value);
    tok.gpool = P.gate;
    tok.row = s_row;
    tok.bs = P.block_size;
    tok.H = P.H;
    tok.h = h;
    tok.p = p;
    tok.kin = static_cast<const IO*>(P.k) + in_row * DK;
    tok.vin = static_cast<const IO*>(P.v) + in_row * DV;
    tok.gin = GATED ? P.g + in_row : nullptr;
    tok.in_stride_k = static_cast<size_t>(P.H) * DK;
    tok.in_stride_v = static_cast<size_t>(P.H) * DV;

    if (token_wave) {
        // ---- token wave ------------------------------------------------------
        // (s_row was written by lane 0 of this wave; the LDS operations of one
        // wave complete in order.)  Sixteen lanes share a token row: lane
        // group gl (0..3) takes one position per round, lane cl (0..15) one
        // E-element chunk of it.  All loads of a batch of 8 positions are
        // issued before any is used: one HBM round trip per batch.
        constexpr int E = G::E, EV = DV / 16, NB = 2, NQR = (NQ + 3) / 4;
        const int gl = lane >> 4, cl = lane & 15;
        // queries (and, delta rule, keys) of this call's tokens
        RawChunk<IO, E> qraw[NQR], kdraw[DELTA ? NQR : 1];
#pragma unroll
        for (int r = 0; r < NQR; ++r) {
            const int d = gl + 4 * r;
            qraw[r].zero();
            if constexpr (DELTA) kdraw[r].zero();
            if (d < n) {
                qraw[r].load(static_cast<const IO*>(P.q) + (in_row + d * P.H) * DK + cl * E);
                if constexpr (DELTA) kdraw[r].load(tok.kin + d * tok.in_stride_k + cl * E);
            }
        }
        float accq[NQ][EV], acck[DELTA ? NQ : 1][EV];
#pragma unroll
        for (int d = 0; d < NQ; ++d)
#pragma unroll
            for (int e = 0; e < EV; ++e) {
                accq[d][e] = 0.f;
                if constexpr (DELTA) acck[d][e] = 0.f;
            }
        const int tacc = DELTA ? p : T;  // positions whose values enter the sums
        const int nfold = fold ? P.m : 0;  // positions staged for the fold
        IO* kpool = static_cast<IO*>(P.key);
        XIO* xpool = static_cast<XIO*>(P.value);
        for (int i0 = 0; i0 < T; i0 += 4 * NB) {
            RawChunk<IO, E> kr[NB];
            RawChunk<XIO, EV> xr[NB];
#pragma unroll
            for (int rr = 0; rr < NB; ++rr) {
                const int i = i0 + 4 * rr + gl;
                kr[rr].zero();
                xr[rr].zero();
                if (i < T) {
                    kr[rr].load(tok.key(i) + cl * E);
                    if (i < p) {
                        xr[rr].load(tok.pooled_value(i) + cl * EV);
                    } else if constexpr (!DELTA) {
                        xr[rr].load(tok.new_value(i - p) + cl * EV);
                    }
                }
            }
            if (i0 == 0) {
                // gate prefix sums (their loads join this round trip), then
                // the queries to LDS
                if constexpr (GATED) {
                    gate_prefix(bl, T, lane, [&](int i) { return tok.gate(i); });
                } else {
                    for (int i = lane; i < T; i += 64) bl[i] = 0.0f;
                }
                if (lane < n) es[lane] = GATED ? expf(bl[p + lane]) : 1.0f;
                if (fold && lane == 0) es[NQ] = GATED ? expf(bl[P.m - 1]) : 1.0f;
#pragma unroll
                for (int r = 0; r < NQR; ++r) {
                    const int d = gl + 4 * r;
                    if (d < n) {
                        float f[E];
                        qraw[r].to_float(f);
#pragma unroll
                        for (int e = 0; e < E; ++e) qs[d * DK + cl * E + e] = P.scale * f[e];
                        if constexpr (DELTA) {
                            kdraw[r].to_float(f);
#pragma unroll
                            for (int e = 0; e < E; ++e) ks[d * DK + cl * E + e] = f[e];
                        }
                    }
                }
            }
#pragma unroll
            for (int rr = 0; rr < NB; ++rr) {
                const int i = i0 + 4 * rr + gl;
                const int ic = min(i, T - 1);
                float kf[E], xf[EV];
                kr[rr].to_float(kf);
                xr[rr].to_float(xf);
#pragma unroll
                for (int d = 0; d < NQ; ++d) {
                    if (d < n) {
                        const int t = p + d;
                        float part = 0.f;
#pragma unroll
                        for (int e = 0; e < E; ++e) part += qs[d * DK + cl * E + e] * kf[e];
                        const float dot = group16_sum(part);
                        const float wq = (i <= t) ? (GATED ? expf(bl[t] - bl[ic]) : 1.0f) * dot : 0.f;
                        if (cl == 0 && i < T) cq[d * ldc + i] = wq;
                        if (i < tacc) {
#pragma unroll
                            for (int e = 0; e < EV; ++e) accq[d][e] += wq * xf[e];
                        }
                        if constexpr (DELTA) {
                            float pk = 0.f;
#pragma unroll
                            for (int e = 0; e < E; ++e) pk += ks[d * DK + cl * E + e] * kf[e];
                            const float dk = group16_sum(pk);
                            const float wk = (i < t) ? (GATED ? expf(bl[t] - bl[ic]) : 1.0f) * dk : 0.f;
                            if (cl == 0 && i < T) ck[d * ldc + i] = wk;
                            if (i < tacc) {
#pragma unroll
                                for (int e = 0; e < EV; ++e) acck[d][e] += wk * xf[e];
                            }
                        }
                    }
                }
                // the same registers feed the fold staging and the appends
                if (i < nfold) {
#pragma unroll
                    for (int e = 0; e < E; ++e) fk[i * DK + cl * E + e] = kf[e];
                    if (!DELTA || i < p) {
#pragma unroll
                        for (int e = 0; e < EV; ++e) fx[i * DV + cl * EV + e] = xf[e];
                    }
                }
                if (i >= p && i < T) {
                    kr[rr].store(kpool + tok.slot_index(i) * DK + cl * E);
                    if constexpr (!DELTA) xr[rr].store(xpool + tok.slot_index(i) * DV + cl * EV);
                }
            }
        }
        // sum the four position groups; group 0 writes the totals
#pragma unroll
        for (int d = 0; d < NQ; ++d) {
            if (d < n) {
#pragma unroll
                for (int e = 0; e < EV; ++e) {
                    float v = accq[d][e];
                    v += __shfl_xor(v, 16, 64);
                    v += __shfl_xor(v, 32, 64);
                    if (gl == 0) lds[L.bq + d * DV + cl * EV + e] = v;
                    if constexpr (DELTA) {
                        float vk = acck[d][e];
                        vk += __shfl_xor(vk, 16, 64);
                        vk += __shfl_xor(vk, 32, 64);
                        if (gl == 0) lds[L.bk + d * DV + cl * EV + e] = vk;
                    }
                }
            }
        }
        for (int ii = lane; ii < nfold; ii += 64) fw[ii] = GATED ? expf(bl[P.m - 1] - bl[ii]) : 1.0f;
        if constexpr (GATED) {
            if (lane < n) P.gate[tok.slot_index(p + lane)] = tok.gin[lane * P.H];
        }
    }
    // ---- state waves: put the whole tile in flight ------------------------------
    // (After the token-wave block in program order, so that none of the token
    // wave's registers are allocated on top of the tile's 64.)
    f4 s[RPT];
    if (!token_wave && has_state) {
        const float* stile = P.state + (static_cast<size_t>(slot) * P.H + h) * DK * DV;
#pragma unroll
        for (int j = 0; j < RPT; ++j)
            s[j] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(stile + (rg + RG * j) * DV + c0));
    }
    __syncthreads();
    // Every wave is past its reads of the request's metadata.
    const bool advance = P.mode != MODE_VERIFY;  // drafts do not advance the occupancy
    if (advance && tid == NT) s_last = take_ticket(P, b);

    // ---- S^T q (and S^T k) from the state registers, reduced over row groups
    float* red = lds + L.red;
    float* outp = P.out + in_row * DV;
    const size_t out_stride = static_cast<size_t>(P.H) * DV;
#pragma unroll
    for (int d = 0; d < NQ; ++d) {
        if (d < n) {
            if (!token_wave) {
                f4 a = f4{0.f, 0.f, 0.f, 0.f};
                f4 ak = f4{0.f, 0.f, 0.f, 0.f};
                if (has_state) {
#pragma unroll
                    for (int j = 0; j < RPT; ++j) {
                        a += s[j] * qs[d * DK + rg + RG * j];
                        if constexpr (DELTA) ak += s[j] * ks[d * DK + rg + RG * j];
                    }
                }
                *reinterpret_cast<f4*>(red + rg * DV + c0) = a * es[d];
                if constexpr (DELTA) *reinterpret_cast<f4*>(red + (RG + rg) * DV + c0) = ak * es[d];
            }
            __syncthreads();
            for (int c = tid; c < DV; c += G::NTHREADS) {
                float sum = lds[L.bq + d * DV + c];
                float sumk = DELTA ? lds[L.bk + d * DV + c] : 0.f;
#pragma unroll
                for (int g2 = 0; g2 < RG; ++g2) {
                    sum += red[g2 * DV + c];
                    if constexpr (DELTA) sumk += red[(RG + g2) * DV + c];
                }
                if constexpr (DELTA) {
                    lds[L.sq + d * DV + c] = sum;
                    lds[L.sk + d * DV + c] = sumk;
                } else {
                    outp[d * out_stride + c] = sum;
                }
            }
            __syncthreads();
        }
    }

    // ---- delta rule: pseudo-values and outputs of the new tokens -------------
    if constexpr (DELTA) {
        XIO* xpool = static_cast<XIO*>(P.value);
        for (int c = tid; c < DV; c += G::NTHREADS) {
            float u[NQ];
#pragma unroll
            for (int d = 0; d < NQ; ++d) {
                u[d] = 0.f;
                if (d < n) {
                    const int t = p + d;
                    float x = load1(tok.new_value(d) + c) - lds[L.sk + d * DV + c];
                    float o = lds[L.sq + d * DV + c];
#pragma unroll
                    for (int e = 0; e < d; ++e) x -= ck[d * ldc + p + e] * u[e];
                    x *= P.beta[in_row + static_cast<size_t>(d) * P.H];
                    u[d] = x;
#pragma unroll
                    for (int e = 0; e <= d; ++e) o += cq[d * ldc + p + e] * u[e];
                    outp[d * out_stride + c] = o;
                    lds[L.un + d * DV + c] = x;
                    xpool[tok.slot_index(t) * DV + c] = x;
                    if (fold && t < P.m) fx[t * DV + c] = x;  // the new token is folded too
                }
            }
        }
        __syncthreads();
    }

    // ---- eager fold: the buffer reached m tokens -----------------------------
    // All m tokens were staged by the token wave (m <= fold_chunk: the
    // launcher only lets this kernel fold when they fit one staging round).
    if (fold) {
        if (!token_wave) {
            const float e0 = es[NQ];
#pragma unroll
            for (int j = 0; j < RPT; ++j) s[j] *= e0;
            for (int ii = 0; ii < P.m; ++ii) {
                const f4 x = *reinterpret_cast<const f4*>(fx + ii * DV + c0);
                const float w = fw[ii];
#pragma unroll
                for (int j = 0; j < RPT; ++j) s[j] += (w * fk[ii * DK + rg + RG * j]) * x;
            }
            float* wt = P.state + (static_cast<size_t>(slot) * P.H + h) * DK * DV;
#pragma unroll
            for (int j = 0; j < RPT; ++j)
                __builtin_nontemporal_store(s[j], reinterpret_cast<f4*>(wt + (rg + RG * j) * DV + c0));
        }
    }

    // ---- bookkeeping -----------------------------------------------------------
    if (!advance) return;
    __syncthreads();
    apply_bookkeeping(P, b, s_last, T - (fold ? P.m : 0), fold ? P.m / P.block_size : 0);
}

template <int RULE, int D, typename IO>
hipError_t launch_chunk_t(const TileParams& p, int batch, hipStream_t s) {
    using G = Geo<D, D>;
    const int cap = p.block_size * p.blocks_per_req;
    const int nq = p.n <= 1 ? 1 : p.n <= 2 ? 2 : p.n <= 4 ? 4 : 8;
    const size_t lds = sizeof(float) * chunk_lds(RULE, D, D, nq, G::RG, cap, p.fold_chunk).total;
    const dim3 grid(static_cast<unsigned>(batch) * p.H), block(G::NTHREADS);
    switch (nq) {
        case 1: chunk_kernel<RULE, D, D, 1, IO><<<grid, block, lds, s>>>(p); break;
        case 2: chunk_kernel<RULE, D, D, 2, IO><<<grid, block, lds, s>>>(p); break;
        case 4: chunk_kernel<RULE, D, D, 4, IO><<<grid, block, lds, s>>>(p); break;
        default: chunk_kernel<RULE, D, D, 8, IO><<<grid, block, lds, s>>>(p); break;
    }
    return hipGetLastError();
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

hipError_t launch_chunk(const TileParams& p, int rule, int d, int io, int batch, hipStream_t s) {
    return io == KVBUF_BF16 ? launch_chunk_r<bf16_bits>(p, rule, d, batch, s)
                            : launch_chunk_r<float>(p, rule, d, batch, s);
}

}  // namespace kvbuf
