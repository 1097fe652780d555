// Recurrent decode: the buffer size m = 0 case.
//
// KVBuffer: IO-aware Serving for Linear Attention (pith.science page,
// abstract: existing serving systems recompute and update the whole state at
// every decoding step; Figure 3 caption: this is the m = 0 baseline the
// buffered kernels are normalised by).  Per token and (request, head):
//   linear   S <- S + k v^T
//   gated    S <- e^g S + k v^T
//   delta    S <- e^g S + k u^T,  u = beta (v - e^g S^T k)
//            (the same as e^g (I - beta k k^T) S + beta k v^T)
//   channel  S <- diag(e^g) S + k v^T, one log-gate per key channel (row)
//   output   o = S^T (scale q) with the updated S.
// One workgroup per tile reads the 64 KiB state once and writes it once:
// 2 |S| bytes of HBM traffic per token, which is what the buffered path avoids.
// As in the buffered kernels, the state waves put the tile in flight while
// the token wave stages q, k, v and the gate.
#include "device_common.hpp"

namespace kvbuf {
namespace {

template <int RULE, int DK, int DV, typename IO>
__global__ __launch_bounds__((Geo<DK, DV>::NTHREADS)) void recurrent_kernel(TileParams P) {
    using G = Geo<DK, DV>;
    constexpr int NT = G::NT, TPR = G::TPR, RG = G::RG, RPT = G::RPT;
    constexpr bool DELTA = RULE == KVBUF_RULE_DELTA;
    constexpr bool CH = RULE == KVBUF_RULE_CHANNEL;
    constexpr bool GATED = RULE != KVBUF_RULE_LINEAR;

    __shared__ float qs[DK];
    __shared__ float kf[DK];
    __shared__ float vf[DV];
    __shared__ float red[RG * DV];
    __shared__ float sk[DELTA ? DV : 1];
    __shared__ float gb[2];           // gamma, beta
    __shared__ float gv[CH ? DK : 1];  // per-channel decay e^{g[r]}

    const TileIndex ti = tile_index(P);
    const int b = ti.b;
    const int h = ti.h;
    const int tid = threadIdx.x;
    const bool token_wave = tid >= NT;
    const int lane = tid - NT;
    const int rg = tid / TPR;
    const int c0 = (tid % TPR) * 4;

    const int slot = P.slot[b];
    if (slot < 0 || slot >= P.num_slots) {
        report(P, KVBUF_DEVERR_SLOT);
        return;
    }
    float* stile = P.state + (static_cast<size_t>(slot) * P.H + h) * DK * DV;
    const size_t in_row = static_cast<size_t>(b) * P.H + h;
    if (token_wave) {
        const IO* q = static_cast<const IO*>(P.q) + in_row * DK;
        const IO* k = static_cast<const IO*>(P.k) + in_row * DK;
        const IO* v = static_cast<const IO*>(P.v) + in_row * DV;
        for (int r = lane; r < DK; r += 64) {
            qs[r] = P.scale * load1(q + r);
            kf[r] = load1(k + r);
        }
        for (int c = lane; c < DV; c += 64) vf[c] = load1(v + c);
        if constexpr (CH) {
            for (int r = lane; r < DK; r += 64) gv[r] = exp_gate(P.g[in_row * DK + r]);
        }
        if (lane == 0) {
            gb[0] = (GATED && !CH) ? exp_gate(P.g[in_row]) : 1.0f;
            gb[1] = DELTA ? P.beta[in_row] : 0.0f;
        }
    }
    // (after the token-wave block, so its registers are not allocated on top
    // of the tile's)
    f4 s[RPT];
    if (!token_wave) {
#pragma unroll
        for (int j = 0; j < RPT; ++j)
            s[j] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(stile + (rg * RPT + j) * DV + c0));
    }
    __syncthreads();
    const float gamma = gb[0];
    f4 x = *reinterpret_cast<const f4*>(vf + c0);

    if constexpr (DELTA) {
        if (!token_wave) {
            f4 a = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < RPT; ++j) a += s[j] * kf[rg * RPT + j];
            *reinterpret_cast<f4*>(red + rg * DV + c0) = a;
        }
        __syncthreads();
        for (int c = tid; c < DV; c += G::NTHREADS) {
            float sum = 0.f;
#pragma unroll
            for (int g2 = 0; g2 < RG; ++g2) sum += red[g2 * DV + c];
            sk[c] = sum;
        }
        __syncthreads();
        const f4 skv = *reinterpret_cast<const f4*>(sk + c0);
        x = gb[1] * (x - gamma * skv);
    }

    if (!token_wave) {
        f4 o = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const int r = rg * RPT + j;
            s[j] = (CH ? gv[r] : gamma) * s[j] + kf[r] * x;
            o += s[j] * qs[r];
        }
#pragma unroll
        for (int j = 0; j < RPT; ++j)
            __builtin_nontemporal_store(s[j], reinterpret_cast<f4*>(stile + (rg * RPT + j) * DV + c0));
        *reinterpret_cast<f4*>(red + rg * DV + c0) = o;
    }
    __syncthreads();
    for (int c = tid; c < DV; c += G::NTHREADS) {
        float sum = 0.f;
#pragma unroll
        for (int g2 = 0; g2 < RG; ++g2) sum += red[g2 * DV + c];
        store_out(P, in_row * DV + c, sum);
    }
}

// Verification with temporary states: drafts d = 0..n-1 of request b are
// applied one at a time to a copy of its state, with the same per-token
// update as above; draft d's output and the state after it (a temporary
// state, temp [n][B][H][d_k][d_v]) are written out.  One state read, n state
// writes per tile.  The token wave stages all n drafts first.
template <int RULE, int DK, int DV, typename IO>
__global__ __launch_bounds__((Geo<DK, DV>::NTHREADS)) void verify_recurrent_kernel(TileParams P, float* temp) {
    using G = Geo<DK, DV>;
    constexpr int NT = G::NT, TPR = G::TPR, RG = G::RG, RPT = G::RPT;
    constexpr int NMAX = kMaxDrafts;
    constexpr bool DELTA = RULE == KVBUF_RULE_DELTA;
    constexpr bool CH = RULE == KVBUF_RULE_CHANNEL;
    constexpr bool GATED = RULE != KVBUF_RULE_LINEAR;

    __shared__ float qs[NMAX][DK];
    __shared__ float kf[NMAX][DK];
    __shared__ float vf[NMAX][DV];
    __shared__ float gb[NMAX][2];  // gamma, beta
    __shared__ float gv[CH ? NMAX : 1][CH ? DK : 1];  // per-channel decays of each draft
    __shared__ float red[2][RG * DV];
    __shared__ float sk[DELTA ? DV : 1];

    const TileIndex ti = tile_index(P);
    const int b = ti.b;
    const int h = ti.h;
    const int n = P.n;
    const int tid = threadIdx.x;
    const bool token_wave = tid >= NT;
    const int lane = tid - NT;
    const int rg = tid / TPR;
    const int c0 = (tid % TPR) * 4;

    const int slot = P.slot[b];
    if (slot < 0 || slot >= P.num_slots) {
        report(P, KVBUF_DEVERR_SLOT);
        return;
    }
    const float* stile = P.state + (static_cast<size_t>(slot) * P.H + h) * DK * DV;
    if (token_wave) {
        for (int d = 0; d < n; ++d) {
            const size_t row = (static_cast<size_t>(b) * n + d) * P.H + h;  // [B][n][H]
            const IO* q = static_cast<const IO*>(P.q) + row * DK;
            const IO* k = static_cast<const IO*>(P.k) + row * DK;
            const IO* v = static_cast<const IO*>(P.v) + row * DV;
            for (int r = lane; r < DK; r += 64) {
                qs[d][r] = P.scale * load1(q + r);
                kf[d][r] = load1(k + r);
            }
            for (int c = lane; c < DV; c += 64) vf[d][c] = load1(v + c);
            if constexpr (CH) {
                for (int r = lane; r < DK; r += 64) gv[d][r] = exp_gate(P.g[row * DK + r]);
            }
            if (lane == 0) {
                gb[d][0] = (GATED && !CH) ? exp_gate(P.g[row]) : 1.0f;
                gb[d][1] = DELTA ? P.beta[row] : 0.0f;
            }
        }
    }
    f4 s[RPT];
    if (!token_wave) {
#pragma unroll
        for (int j = 0; j < RPT; ++j)
            s[j] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(stile + (rg * RPT + j) * DV + c0));
    }
    __syncthreads();

    for (int d = 0; d < n; ++d) {
        float* rd = red[d & 1];  // alternate buffers: one barrier per draft
        const float gamma = gb[d][0];
        f4 x = *reinterpret_cast<const f4*>(&vf[d][c0]);
        if constexpr (DELTA) {
            if (!token_wave) {
                f4 a = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < RPT; ++j) a += s[j] * kf[d][rg * RPT + j];
                *reinterpret_cast<f4*>(rd + rg * DV + c0) = a;
            }
            __syncthreads();
            for (int c = tid; c < DV; c += G::NTHREADS) {
                float sum = 0.f;
#pragma unroll
                for (int g2 = 0; g2 < RG; ++g2) sum += rd[g2 * DV + c];
                sk[c] = sum;
            }
            __syncthreads();
            x = gb[d][1] * (x - gamma * *reinterpret_cast<const f4*>(sk + c0));
            rd = red[(d + 1) & 1];
        }
        if (!token_wave) {
            f4 o = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < RPT; ++j) {
                const int r = rg * RPT + j;
                s[j] = (CH ? gv[d][r] : gamma) * s[j] + kf[d][r] * x;
                o += s[j] * qs[d][r];
            }
            float* tt = temp + ((static_cast<size_t>(d) * P.batch + b) * P.H + h) * DK * DV;
#pragma unroll
            for (int j = 0; j < RPT; ++j)
                __builtin_nontemporal_store(s[j], reinterpret_cast<f4*>(tt + (rg * RPT + j) * DV + c0));
            *reinterpret_cast<f4*>(rd + rg * DV + c0) = o;
        }
        __syncthreads();
        const size_t orow = (static_cast<size_t>(b) * n + d) * P.H + h;
        for (int c = tid; c < DV; c += G::NTHREADS) {
            float sum = 0.f;
#pragma unroll
            for (int g2 = 0; g2 < RG; ++g2) sum += rd[g2 * DV + c];
            store_out(P, orow * DV + c, sum);
        }
        if constexpr (DELTA) __syncthreads();  // sk and both partial buffers are reused
    }
}

// Commit of the recurrent verification: state[slot] <- temp[a - 1].
template <int DK, int DV>
__global__ __launch_bounds__(256) void commit_recurrent_kernel(TileParams P, const float* temp) {
    const TileIndex ti = tile_index(P);
    const int b = ti.b;
    const int h = ti.h;
    const int a = P.accepted[b];
    const int slot = P.slot[b];
    if (a < 0 || a > P.n) {
        report(P, KVBUF_DEVERR_ACCEPT);
        return;
    }
    if (slot < 0 || slot >= P.num_slots) {
        report(P, KVBUF_DEVERR_SLOT);
        return;
    }
    if (a == 0) return;
    const f4* src = reinterpret_cast<const f4*>(temp + ((static_cast<size_t>(a - 1) * P.batch + b) * P.H + h) * DK * DV);
    f4* dst = reinterpret_cast<f4*>(P.state + (static_cast<size_t>(slot) * P.H + h) * DK * DV);
    constexpr int N4 = DK * DV / 4;
    constexpr int PER = (N4 + 255) / 256;
    f4 buf[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = threadIdx.x + 256 * i;
        if (e < N4) buf[i] = __builtin_nontemporal_load(src + e);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = threadIdx.x + 256 * i;
        if (e < N4) __builtin_nontemporal_store(buf[i], dst + e);
    }
}

template <int RULE, int D, typename IO>
hipError_t launch_rec_t(const TileParams& p, int batch, hipStream_t s) {
    using G = Geo<D, D>;
    recurrent_kernel<RULE, D, D, IO><<<dim3(static_cast<unsigned>(batch) * p.H), dim3(G::NTHREADS), 0, s>>>(p);
    return hipGetLastError();
}

template <int RULE, typename IO>
hipError_t launch_rec_d(const TileParams& p, int d, int batch, hipStream_t s) {
    switch (d) {
        case 16: return launch_rec_t<RULE, 16, IO>(p, batch, s);
        case 64: return launch_rec_t<RULE, 64, IO>(p, batch, s);
        default: return launch_rec_t<RULE, 128, IO>(p, batch, s);
    }
}

template <typename IO>
hipError_t launch_rec_r(const TileParams& p, int rule, int d, int batch, hipStream_t s) {
    switch (rule) {
        case KVBUF_RULE_LINEAR: return launch_rec_d<KVBUF_RULE_LINEAR, IO>(p, d, batch, s);
        case KVBUF_RULE_GATED: return launch_rec_d<KVBUF_RULE_GATED, IO>(p, d, batch, s);
        case KVBUF_RULE_CHANNEL: return launch_rec_d<KVBUF_RULE_CHANNEL, IO>(p, d, batch, s);
        default: return launch_rec_d<KVBUF_RULE_DELTA, IO>(p, d, batch, s);
    }
}

template <int RULE, int D, typename IO>
hipError_t launch_verify_rec_t(const TileParams& p, float* temp, hipStream_t s) {
    using G = Geo<D, D>;
    verify_recurrent_kernel<RULE, D, D, IO><<<dim3(static_cast<unsigned>(p.batch) * p.H), dim3(G::NTHREADS), 0, s>>>(p, temp);
    return hipGetLastError();
}

template <int RULE, typename IO>
hipError_t launch_verify_rec_d(const TileParams& p, int d, float* temp, hipStream_t s) {
    switch (d) {
        case 16: return launch_verify_rec_t<RULE, 16, IO>(p, temp, s);
        case 64: return launch_verify_rec_t<RULE, 64, IO>(p, temp, s);
        default: return launch_verify_rec_t<RULE, 128, IO>(p, temp, s);
    }
}

template <typename IO>
hipError_t launch_verify_rec_r(const TileParams& p, int rule, int d, float* temp, hipStream_t s) {
    switch (rule) {
        case KVBUF_RULE_LINEAR: return launch_verify_rec_d<KVBUF_RULE_LINEAR, IO>(p, d, temp, s);
        case KVBUF_RULE_GATED: return launch_verify_rec_d<KVBUF_RULE_GATED, IO>(p, d, temp, s);
        case KVBUF_RULE_CHANNEL: return launch_verify_rec_d<KVBUF_RULE_CHANNEL, IO>(p, d, temp, s);
        default: return launch_verify_rec_d<KVBUF_RULE_DELTA, IO>(p, d, temp, s);
    }
}

}  // namespace

hipError_t launch_recurrent(const TileParams& p, int rule, int d, int io, int batch, hipStream_t s) {
    return io == KVBUF_BF16 ? launch_rec_r<bf16_bits>(p, rule, d, batch, s)
                            : launch_rec_r<float>(p, rule, d, batch, s);
}

hipError_t launch_verify_recurrent(const TileParams& p, int rule, int d, int io, float* temp, hipStream_t s) {
    return io == KVBUF_BF16 ? launch_verify_rec_r<bf16_bits>(p, rule, d, temp, s)
                            : launch_verify_rec_r<float>(p, rule, d, temp, s);
}

hipError_t launch_commit_recurrent(const TileParams& p, int d, const float* temp, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(p.batch) * p.H), block(256);
    switch (d) {
        case 16: commit_recurrent_kernel<16, 16><<<grid, block, 0, s>>>(p, temp); break;
        case 64: commit_recurrent_kernel<64, 64><<<grid, block, 0, s>>>(p, temp); break;
        default: commit_recurrent_kernel<128, 128><<<grid, block, 0, s>>>(p, temp); break;
    }
    return hipGetLastError();
}

}  // namespace kvbuf
