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
// One workgroup per (request, head).  The workgroup issues all loads of its
// 64 KiB state tile first (128-bit, non-temporal: the tile is not reused
// before it is evicted), computes the gates' prefix sums and the q . k scores
// of the buffered tokens while they are in flight, then reduces S^T q and the
// weighted buffer sum in one pass over its registers.  The state is the only
// large operand, so the kernel is bound by HBM bandwidth; everything else is
// sized to stay off that path.
#include "device_common.hpp"

namespace kvbuf {
namespace {

// LDS layout of the chunk kernel, in floats.  Shared by the launcher (size)
// and the kernel (offsets).
struct ChunkLds {
    int qs, ks, bl, cq, ck, es, sq, sk, un, red, fk, fx, fw, total;
};

__host__ __device__ inline int round4(int x) { return (x + 3) & ~3; }

__host__ __device__ inline ChunkLds chunk_lds(int rule, int DK, int DV, int NQ, int RG, int cap, bool fold) {
    ChunkLds L;
    int o = 0;
    const bool delta = rule == KVBUF_RULE_DELTA;
    L.qs = o; o += NQ * DK;                       // scaled queries of the new tokens
    L.ks = o; o += delta ? NQ * DK : 0;           // keys of the new tokens (delta rule)
    L.bl = o; o += round4(cap);                   // cumulative log-gates
    L.cq = o; o += NQ * round4(cap);              // e^{b_t - b_i} (q_t . k_i)
    L.ck = o; o += delta ? NQ * round4(cap) : 0;  // e^{b_t - b_i} (k_t . k_i)
    L.es = o; o += round4(NQ);                    // e^{b_t}, the weight of S0
    L.sq = o; o += delta ? NQ * DV : 0;           // reduced e^{b_t} S0^T q_t + buffer part
    L.sk = o; o += delta ? NQ * DV : 0;           // reduced e^{b_t} S0^T k_t + buffer part
    L.un = o; o += delta ? NQ * DV : 0;           // pseudo-values of the new tokens
    // The row-group reduction area and the fold staging area are never live
    // at the same time.
    const int red = RG * DV * (delta ? 2 : 1);
    const int stage = fold ? kFoldChunk * (DK + DV) + kFoldChunk : 0;
    L.red = o;
    L.fk = o;
    L.fx = o + kFoldChunk * DK;
    L.fw = L.fx + kFoldChunk * DV;
    o += red > stage ? red : stage;
    L.total = o;
    return L;
}

template <int RULE, int DK, int DV, int NQ, typename IO>
__global__ __launch_bounds__((Geo<DK, DV>::NT)) void chunk_kernel(TileParams P) {
    using G = Geo<DK, DV>;
    constexpr int NT = G::NT, TPR = G::TPR, RG = G::RG, RPT = G::RPT;
    constexpr bool DELTA = RULE == KVBUF_RULE_DELTA;
    constexpr bool GATED = RULE != KVBUF_RULE_LINEAR;
    using XIO = typename std::conditional<DELTA, float, IO>::type;

    extern __shared__ float lds[];
    __shared__ int32_t s_row[kMaxTableRow];

    const int tile = blockIdx.x;
    const int b = tile / P.H;
    const int h = tile - b * P.H;
    const int tid = threadIdx.x;
    const int rg = tid / TPR;
    const int c0 = (tid % TPR) * 4;
    const int n = P.n;
    const int cap = P.block_size * P.blocks_per_req;
    const bool direct = P.mode == MODE_DIRECT;

    const int p = P.occ[b];
    const int slot = direct ? -1 : P.slot[b];
    unsigned bad = (p < 0) ? KVBUF_DEVERR_OVERFLOW : load_row(P, b, p + n, s_row);
    if (slot >= P.num_slots) bad |= KVBUF_DEVERR_SLOT;
    if (bad) {
        report(P, bad);
        return;  // the whole request is skipped by all of its workgroups
    }
    const bool has_state = slot >= 0;
    const int T = p + n;  // positions touched by this call
    const bool fold = P.mode == MODE_DECODE && P.fuse && has_state && T >= P.m;

    // ---- 1. issue the state tile loads -----------------------------------
    f4 s[RPT];
    const float* stile = P.state + (static_cast<size_t>(has_state ? slot : 0) * P.H + h) * DK * DV;
    if (has_state) {
#pragma unroll
        for (int j = 0; j < RPT; ++j)
            s[j] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(stile + (rg + RG * j) * DV + c0));
    }

    const ChunkLds L = chunk_lds(RULE, DK, DV, NQ, RG, cap, P.fuse != 0);
    float* qs = lds + L.qs;
    float* ks = lds + L.ks;
    float* bl = lds + L.bl;
    float* cq = lds + L.cq;
    float* ck = lds + L.ck;
    float* es = lds + L.es;
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

    // ---- 2. stage queries (and delta-rule keys) --------------------------
    for (int e = tid; e < n * DK; e += NT) {
        const int d = e / DK, r = e - d * DK;
        qs[d * DK + r] = P.scale * load1(static_cast<const IO*>(P.q) + (in_row + d * P.H) * DK + r);
        if constexpr (DELTA) ks[d * DK + r] = load1(tok.kin + d * tok.in_stride_k + r);
    }
    __syncthreads();  // s_row is complete

    // ---- 3. cumulative log-gates ------------------------------------------
    if constexpr (GATED) {
        gate_prefix(bl, T, [&](int i) { return tok.gate(i); });
    } else {
        for (int i = tid; i < T; i += NT) bl[i] = 0.0f;
    }
    __syncthreads();
    if (tid < n) es[tid] = GATED ? expf(bl[p + tid]) : 1.0f;

    // ---- 4. scores: 16-lane groups, one (draft, position) pair per round --
    {
        const int lane = tid % G::DOT_LANES;
        const int grp = tid / G::DOT_LANES;
        const int npq = n * T;
        const int npairs = DELTA ? 2 * npq : npq;
        for (int pi = grp; pi < npairs; pi += G::GROUPS) {
            const bool kk = DELTA && pi >= npq;
            const int pp = kk ? pi - npq : pi;
            const int d = pp / T;
            const int i = pp - d * T;
            const int t = p + d;  // position of draft d
            const bool live = kk ? (i < t) : (i <= t);
            float part = 0.0f;
            if (live) {
                float kv[G::E];
                loadE<G::E>(tok.key(i) + lane * G::E, kv);
                const float* a = (kk ? ks : qs) + d * DK + lane * G::E;
#pragma unroll
                for (int e = 0; e < G::E; ++e) part += a[e] * kv[e];
            }
            const float dot = group16_sum(part);
            if (lane == 0) {
                const float w = live ? (GATED ? expf(bl[t] - bl[i]) : 1.0f) * dot : 0.0f;
                (kk ? ck : cq)[d * ldc + i] = w;
            }
        }
    }
    __syncthreads();

    // ---- 5. one pass over the state registers + the weighted buffer sum --
    // Rows of this thread: r_j = rg + RG * j; columns c0 .. c0+3.
    f4 acc[NQ];
    f4 acck[DELTA ? NQ : 1];
#pragma unroll
    for (int d = 0; d < NQ; ++d) {
        acc[d] = f4{0.f, 0.f, 0.f, 0.f};
        if constexpr (DELTA) acck[d] = f4{0.f, 0.f, 0.f, 0.f};
    }
    if (has_state) {
#pragma unroll
        for (int d = 0; d < NQ; ++d) {
            if (d < n) {
                f4 a = f4{0.f, 0.f, 0.f, 0.f};
                f4 ak = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < RPT; ++j) {
                    a += s[j] * qs[d * DK + rg + RG * j];
                    if constexpr (DELTA) ak += s[j] * ks[d * DK + rg + RG * j];
                }
                acc[d] = a * es[d];
                if constexpr (DELTA) acck[d] = ak * es[d];
            }
        }
    }
    {
        // Linear / gated: every position including the new tokens (their
        // values are inputs).  Delta: buffered positions only; the new tokens'
        // pseudo-values depend on this reduction and are added in step 7.
        const int tacc = DELTA ? p : T;
        for (int i = rg; i < tacc; i += RG) {
            f4 x = (i < p) ? load4(tok.pooled_value(i) + c0) : load4(tok.new_value(i - p) + c0);
#pragma unroll
            for (int d = 0; d < NQ; ++d) {
                if (d < n) {
                    acc[d] += cq[d * ldc + i] * x;
                    if constexpr (DELTA) acck[d] += ck[d * ldc + i] * x;
                }
            }
        }
    }

    // ---- 6. reduce over row groups ----------------------------------------
    float* red = lds + L.red;
    float* outp = P.out + in_row * DV;
    const size_t out_stride = static_cast<size_t>(P.H) * DV;
#pragma unroll
    for (int d = 0; d < NQ; ++d) {
        if (d < n) {
            *reinterpret_cast<f4*>(red + rg * DV + c0) = acc[d];
            if constexpr (DELTA) *reinterpret_cast<f4*>(red + (RG + rg) * DV + c0) = acck[d];
            __syncthreads();
            for (int c = tid; c < DV; c += NT) {
                float sum = 0.f, sumk = 0.f;
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

    // ---- 7. delta rule: pseudo-values and outputs of the new tokens -------
    if constexpr (DELTA) {
        XIO* xpool = static_cast<XIO*>(P.value);
        for (int c = tid; c < DV; c += NT) {
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
                }
            }
        }
        __syncthreads();
    }

    // ---- 8. eager fold: the buffer reached m tokens ------------------------
    if (fold) {
        const int last = P.m - 1;
        const float e0 = GATED ? expf(bl[last]) : 1.0f;
#pragma unroll
        for (int j = 0; j < RPT; ++j) s[j] *= e0;
        float* fk = lds + L.fk;
        float* fx = lds + L.fx;
        float* fw = lds + L.fw;
        for (int i0 = 0; i0 < P.m; i0 += kFoldChunk) {
            const int cnt = min(kFoldChunk, P.m - i0);
            for (int e = tid; e < cnt * DK; e += NT) {
                const int ii = e / DK, r = e - ii * DK;
                fk[ii * DK + r] = load1(tok.key(i0 + ii) + r);
            }
            for (int e = tid; e < cnt * DV; e += NT) {
                const int ii = e / DV, c = e - ii * DV;
                const int i = i0 + ii;
                float x;
                if (i < p) x = load1(tok.pooled_value(i) + c);
                else if constexpr (DELTA) x = lds[L.un + (i - p) * DV + c];
                else x = load1(tok.new_value(i - p) + c);
                fx[ii * DV + c] = x;
            }
            for (int ii = tid; ii < cnt; ii += NT) fw[ii] = GATED ? expf(bl[last] - bl[i0 + ii]) : 1.0f;
            __syncthreads();
            for (int ii = 0; ii < cnt; ++ii) {
                const f4 x = *reinterpret_cast<const f4*>(fx + ii * DV + c0);
                const float w = fw[ii];
#pragma unroll
                for (int j = 0; j < RPT; ++j) s[j] += (w * fk[ii * DK + rg + RG * j]) * x;
            }
            __syncthreads();
        }
        float* wt = P.state + (static_cast<size_t>(slot) * P.H + h) * DK * DV;
#pragma unroll
        for (int j = 0; j < RPT; ++j)
            __builtin_nontemporal_store(s[j], reinterpret_cast<f4*>(wt + (rg + RG * j) * DV + c0));
    }

    // ---- 9. append the new tokens to the pool ------------------------------
    {
        IO* kpool = static_cast<IO*>(P.key);
        for (int e = tid; e < n * DK; e += NT) {
            const int d = e / DK, r = e - d * DK;
            kpool[tok.slot_index(p + d) * DK + r] = tok.kin[d * tok.in_stride_k + r];
        }
        if constexpr (!DELTA) {
            IO* vpool = static_cast<IO*>(P.value);
            for (int e = tid; e < n * DV; e += NT) {
                const int d = e / DV, c = e - d * DV;
                vpool[tok.slot_index(p + d) * DV + c] = tok.vin[d * tok.in_stride_v + c];
            }
        }
        if constexpr (GATED) {
            if (tid < n) P.gate[tok.slot_index(p + tid)] = tok.gin[tid * P.H];
        }
    }

    // ---- 10. bookkeeping ----------------------------------------------------
    if (P.mode == MODE_VERIFY) return;  // drafts do not advance the occupancy
    finish_request(P, b, T - (fold ? P.m : 0), fold ? P.m / P.block_size : 0);
}

template <int RULE, int D, typename IO>
hipError_t launch_chunk_t(const TileParams& p, int batch, hipStream_t s) {
    using G = Geo<D, D>;
    const int cap = p.block_size * p.blocks_per_req;
    const int nq = p.n <= 1 ? 1 : p.n <= 2 ? 2 : p.n <= 4 ? 4 : 8;
    const size_t lds = sizeof(float) * chunk_lds(RULE, D, D, nq, G::RG, cap, p.fuse != 0).total;
    const dim3 grid(static_cast<unsigned>(batch) * p.H), block(G::NT);
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
