// decode.hip -- single-token recurrent step of the gated delta rule, state updated in place.
//
// One step of "Linear Attention, Visualized", section "Recurrent form", with the decay of
// section "Gated DeltaNet (GDN)" (scalar) or "Kimi Delta Attention (KDA)" (per channel).
// Column convention: S[v][c], v in [0, d_v), c in [0, d_k).
//
// Every row v of S evolves on its own (the transition acts on the key side only), so the
// step is done in ONE pass over the state: with S^ the decayed state,
//     s_k = S^[v,:] . k,   s_q = S^[v,:] . q,   u_v = beta (v_v - s_k),
//     o_v = s_q + u_v (k . q)                (= (S^ + u k^T) q, the read after the write)
//     S[v,:] <- S^[v,:] + u_v k.
// Each row of 4*d_k bytes is held by d_k/4 lanes as float4; a workgroup of eight waves owns
// one (sequence, head) state (d_v/8 rows per wave), issues a batch of row loads before any
// reduction so that many 16-byte requests are in flight, and writes the rows back with
// non-temporal stores: the state is touched once per step and would only pollute L2.  Eight
// waves of d_v/8 rows ran 7% faster than four waves of d_v/4 on the N=256, H=32 shape.
#include "gdr_device.h"

namespace gdr {

constexpr int kDecodeWaves = 8;  // waves per workgroup; d_v (a multiple of 32) splits evenly

template <typename IOT, bool CHANNEL, int DK>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_step_kernel(int dv, const IOT* __restrict__ q,
                                                          const IOT* __restrict__ k,
                                                          const IOT* __restrict__ v,
                                                          const float* __restrict__ g,
                                                          const float* __restrict__ beta,
                                                          float* __restrict__ S, IOT* __restrict__ o) {
    constexpr int LPR = DK / 4;          // lanes per state row
    constexpr int RPI = kWave / LPR;     // rows per wave per instruction
    constexpr int BATCH = 4;             // row-loads in flight per lane (8 waves per SIMD fit)
    const int64_t nh = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane % LPR;          // position inside the row
    const int c0 = sub * 4;

    float kk[4], qq[4], kh[4], qh[4], ach[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        kk[j] = IO<IOT>::load(k, nh * DK + c0 + j);
        qq[j] = IO<IOT>::load(q, nh * DK + c0 + j);
    }
    float a_scalar = 1.0f;
    if constexpr (CHANNEL) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ach[j] = fast_exp(g[nh * DK + c0 + j]);
            kh[j] = ach[j] * kk[j];
            qh[j] = ach[j] * qq[j];
        }
    } else {
        a_scalar = fast_exp(g[nh]);
#pragma unroll
        for (int j = 0; j < 4; ++j) { kh[j] = kk[j]; qh[j] = qq[j]; }
    }
    const float b = beta[nh];
    float kq = kk[0] * qq[0] + kk[1] * qq[1] + kk[2] * qq[2] + kk[3] * qq[3];
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) kq += __shfl_xor(kq, off);

    float* Sh = S + nh * (int64_t)dv * DK;
    const int rows_per_wave = dv / kDecodeWaves;
    const int iters = rows_per_wave / RPI;
    for (int it0 = 0; it0 < iters; it0 += BATCH) {
        float4v row[BATCH];
        const int nb = (iters - it0) < BATCH ? (iters - it0) : BATCH;
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            if (i < nb) {
                const int r = wave * rows_per_wave + (it0 + i) * RPI + lane / LPR;
                row[i] = __builtin_nontemporal_load(reinterpret_cast<const float4v*>(Sh + (int64_t)r * DK + c0));
            }
        }
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            if (i < nb) {
                const int r = wave * rows_per_wave + (it0 + i) * RPI + lane / LPR;
                float4v s = row[i];
                if constexpr (!CHANNEL) s = s * a_scalar;
                float sk = s[0] * kh[0] + s[1] * kh[1] + s[2] * kh[2] + s[3] * kh[3];
                float sq = s[0] * qh[0] + s[1] * qh[1] + s[2] * qh[2] + s[3] * qh[3];
#pragma unroll
                for (int off = LPR / 2; off > 0; off >>= 1) {
                    sk += __shfl_xor(sk, off);
                    sq += __shfl_xor(sq, off);
                }
                const float vv = IO<IOT>::load(v, nh * dv + r);
                const float u = b * (vv - sk);
                if (sub == 0) IO<IOT>::store(o, nh * dv + r, sq + u * kq);
                if constexpr (CHANNEL) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) s[j] = s[j] * ach[j];  // S^[v,c] = S[v,c] a_c
                }
                float4v out;
#pragma unroll
                for (int j = 0; j < 4; ++j) out[j] = s[j] + u * kk[j];
                __builtin_nontemporal_store(out, reinterpret_cast<float4v*>(Sh + (int64_t)r * DK + c0));
            }
        }
    }
}

template <typename IOT, bool CHANNEL, int DK>
static hipError_t launch_decode(int64_t NH, int dv, const void* q, const void* k, const void* v,
                                const float* g, const float* beta, float* S, void* o, hipStream_t st) {
    hipLaunchKernelGGL((decode_step_kernel<IOT, CHANNEL, DK>), dim3((unsigned)NH), dim3(64 * kDecodeWaves), 0, st, dv,
                       (const IOT*)q, (const IOT*)k, (const IOT*)v, g, beta, S, (IOT*)o);
    return hipGetLastError();
}

hipError_t decode_dispatch(int64_t NH, int dk, int dv, bool bf16, bool channel, const void* q, const void* k,
                           const void* v, const float* g, const float* beta, float* S, void* o,
                           hipStream_t st) {
#define GDR_DEC(IOT, CH, DK) return launch_decode<IOT, CH, DK>(NH, dv, q, k, v, g, beta, S, o, st)
    if (bf16) {
        if (channel) { if (dk == 128) GDR_DEC(uint16_t, true, 128); else GDR_DEC(uint16_t, true, 64); }
        else { if (dk == 128) GDR_DEC(uint16_t, false, 128); else GDR_DEC(uint16_t, false, 64); }
    } else {
        if (channel) { if (dk == 128) GDR_DEC(float, true, 128); else GDR_DEC(float, true, 64); }
        else { if (dk == 128) GDR_DEC(float, false, 128); else GDR_DEC(float, false, 64); }
    }
#undef GDR_DEC
}

}  // namespace gdr
