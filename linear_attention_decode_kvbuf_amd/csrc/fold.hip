// Deferred batched state update ("flush"), commit of accepted drafts, and
// materialisation of the effective state.
//
// KVBuffer: IO-aware Serving for Linear Attention (pith.science page):
//  * Figure 1 caption -- when the buffer is full the state is updated with
//    all buffered keys and values on the GPU and written back to the
//    request's state slot;
//  * abstract -- state updates are deferred and applied in batch;
//  * Figure 2 caption -- after verification only the accepted drafts are kept.
//
// Folding positions 0 .. T-1 (cumulative log-gates b_i since the last fold)
// into the state S0 at the last fold:
//   S <- e^{b_{T-1}} S0 + sum_{i<T} e^{b_{T-1} - b_i} k_i x_i^T
// a rank-T update of the d_k x d_v tile (x_i = v_i, or the delta rule's
// pseudo-value u_i).  One workgroup per (request, head): read the 64 KiB tile,
// apply the update from keys and values staged in LDS, write it back.  For
// the buffer sizes served here the update costs 2 T flops per 8 bytes of
// state traffic -- below the fp32 vector ridge of the chip -- so it runs on
// the vector ALUs and the kernel is bound by HBM bandwidth.
#include "device_common.hpp"

namespace kvbuf {
namespace {

__host__ __device__ inline int fold_lds_floats(int DK, int DV, int cap) {
    return ((cap + 3) & ~3) + kFoldChunk * (DK + DV) + kFoldChunk;
}

template <int RULE, int DK, int DV, typename IO>
__global__ __launch_bounds__((Geo<DK, DV>::NT)) void fold_kernel(TileParams P) {
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
    const int cap = P.block_size * P.blocks_per_req;
    const bool materialize = P.mode == MODE_MATERIALIZE;

    const int p = P.occ[b];
    const int slot = P.slot[b];
    unsigned bad = 0;
    int a = 0;
    if (P.mode == MODE_COMMIT) {
        a = P.accepted[b];
        if (a < 0 || a > P.n) bad |= KVBUF_DEVERR_ACCEPT;
    }
    const int pn = p + a;
    if (p < 0 || pn > cap) bad |= KVBUF_DEVERR_OVERFLOW;
    if (slot >= P.num_slots) bad |= KVBUF_DEVERR_SLOT;
    const bool has_state = slot >= 0;
    const bool fold = !materialize && has_state && P.m > 0 && pn >= P.m &&
                      (P.mode == MODE_FLUSH || P.fuse);
    const int T = materialize ? p : (fold ? P.m : 0);  // positions applied
    if (!bad) bad |= load_row(P, b, T, s_row);
    if (bad) {
        report(P, bad);
        return;
    }
    if (!materialize && !fold && a == 0) return;  // nothing changes for this request

    if (materialize || fold) {
        f4 s[RPT];
        const float* stile = P.state + (static_cast<size_t>(has_state ? slot : 0) * P.H + h) * DK * DV;
#pragma unroll
        for (int j = 0; j < RPT; ++j)
            s[j] = has_state ? __builtin_nontemporal_load(reinterpret_cast<const f4*>(stile + (rg + RG * j) * DV + c0))
                             : f4{0.f, 0.f, 0.f, 0.f};

        float* bl = lds;
        float* fk = lds + ((cap + 3) & ~3);
        float* fx = fk + kFoldChunk * DK;
        float* fw = fx + kFoldChunk * DV;

        TileTokens<DK, DV, IO, XIO> tok;
        tok.kpool = static_cast<const IO*>(P.key);
        tok.xpool = static_cast<const XIO*>(P.value);
        tok.gpool = P.gate;
        tok.row = s_row;
        tok.bs = P.block_size;
        tok.H = P.H;
        tok.h = h;
        tok.p = cap;  // every position read here is in the pool

        __syncthreads();  // s_row is complete
        if constexpr (GATED) gate_prefix(bl, T, [&](int i) { return tok.gate(i); });
        __syncthreads();
        if (T > 0) {
            const int last = T - 1;
            const float e0 = GATED ? expf(bl[last]) : 1.0f;
#pragma unroll
            for (int j = 0; j < RPT; ++j) s[j] *= e0;
            for (int i0 = 0; i0 < T; i0 += kFoldChunk) {
                const int cnt = min(kFoldChunk, T - i0);
                for (int e = tid; e < cnt * DK; e += NT) {
                    const int ii = e / DK, r = e - ii * DK;
                    fk[ii * DK + r] = load1(tok.key(i0 + ii) + r);
                }
                for (int e = tid; e < cnt * DV; e += NT) {
                    const int ii = e / DV, c = e - ii * DV;
                    fx[ii * DV + c] = load1(tok.pooled_value(i0 + ii) + c);
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
        }
        float* dst = materialize ? P.states_out + (static_cast<size_t>(b) * P.H + h) * DK * DV
                                 : P.state + (static_cast<size_t>(slot) * P.H + h) * DK * DV;
#pragma unroll
        for (int j = 0; j < RPT; ++j)
            __builtin_nontemporal_store(s[j], reinterpret_cast<f4*>(dst + (rg + RG * j) * DV + c0));
    }

    if (materialize) return;
    finish_request(P, b, pn - (fold ? P.m : 0), fold ? P.m / P.block_size : 0);
}

template <int RULE, int D, typename IO>
hipError_t launch_fold_t(const TileParams& p, int batch, hipStream_t s) {
    using G = Geo<D, D>;
    const size_t lds = sizeof(float) * fold_lds_floats(D, D, p.block_size * p.blocks_per_req);
    fold_kernel<RULE, D, D, IO><<<dim3(static_cast<unsigned>(batch) * p.H), dim3(G::NT), lds, s>>>(p);
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
        default: return launch_fold_d<KVBUF_RULE_DELTA, IO>(p, d, batch, s);
    }
}

}  // namespace

hipError_t launch_fold(const TileParams& p, int rule, int d, int io, int batch, hipStream_t s) {
    return io == KVBUF_BF16 ? launch_fold_r<bf16_bits>(p, rule, d, batch, s)
                            : launch_fold_r<float>(p, rule, d, batch, s);
}

}  // namespace kvbuf
