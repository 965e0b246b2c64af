// chunk_kda.hip -- chunked forward of the gated delta rule with a per-channel gate
// (KDA-style), bf16 I/O, fp16 MFMA operands, fp32 accumulation and state, gfx950.
//
// "Linear Attention, Visualized", sections "Kimi Delta Attention (KDA)" and "Reuse GLA and
// GDN": the decay a_t is a vector over the key channels and acts on S before the delta
// correction, S_t = S_{t-1} Diag(a_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T.  Per chunk,
// with G the in-chunk cumulative log-decay of every (token, channel) and column convention:
//
//   L[l][m] = sum_c k_lc k_mc e^{G_lc - G_mc}   (m < l),   A[l][m] = the same with q_l (m <= l)
//   N = I + diag(beta) L,   T = N^{-1} diag(beta)
//   R = V - (K (.) e^G) S^T,   Z = T R,   O = (Q (.) e^G) S^T + A Z
//   S^T <- Diag(e^{G_C}) S^T + (K (.) e^{G_C - G})^T Z
//
// The decay sits inside the channel sum, so the Gram products take it on their operands:
//   off-diagonal 16x16 tiles (row block bi > column block bj), reference = end of block bj:
//     row operand  K_l e^{G_l - G_start(bi)}            ("Kr", <= 1, one copy of K and Q)
//     column       K_m e^{G_end(bj) - G_m}              ("Kc", <= 1)
//     times the per-channel factor e^{G_start(bi) - G_end(bj)} (<= 1) on the column fragment;
//   diagonal tiles, reference = token 8 of the block: Kr and Kc times e^{-G_loc(8)} and
//     e^{G_loc(8) - G_loc(15)}, per channel (G_loc = cumulative log-decay from the block
//     start).  Those factors exceed 1 by up to e^{8|g|}.  While every |G_loc(t) - G_loc(8)|
//     (t = -1..15, G_loc(-1) = 0) stays within 6 the fp16 path is exact to fp16 rounding;
//     a block beyond that forms its diagonal operands afresh from the bf16 inputs in fp32
//     (e^{G_loc(l) - G_loc(8)} k_l, e^{G_loc(8) - G_loc(m)} k_m) and multiplies them on bf16
//     MFMA, whose exponent range covers any decay the fp32 gate can express.
// After the Gram products the copies are rescaled in place to K (.) e^G, Q (.) e^G and
// K (.) e^{G_C - G} for the state pass (per-block, per-channel factors <= 1).
//
// One workgroup (four waves) per (batch*head, 32-wide d_v tile) walks the chunks in order;
// each chunk runs stage by stage with all waves: scan, staging, Gram, the blocked inverse
// (as in the scalar kernel), then the state pass on waves 0-1.  Loads of chunk c+1 are in
// flight while chunk c is processed.
#include "chunk_common.h"

namespace gdr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct KdaArgs {
    int64_t T;
    int dv;
    int ntiles;  // d_v / 32
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* g;  // [.., T, DK]
    const float* beta;
    const float* S0;
    uint16_t* o;
    float* Sf;
};

template <int DK>
struct KdaLds {
    static constexpr int C = kChunk;
    static constexpr int LDK = DK + 8;   // halfs, rows of the K / Q operand copies
    static constexpr int LDC = C + 8;    // halfs, rows of C-wide fp16 matrices
    static constexpr int LDV = C + 4;    // floats, rows of V^T
    static constexpr int LDN = 16 + 4;   // floats, rows of a 16x16 fp32 block
    static constexpr int LDO = C + 8;    // bf16, rows of O^T
    static constexpr int LDG = DK + 4;   // floats, rows of the block-local cumulative log-decay
    static constexpr int szK = C * LDK * 2;
    static constexpr int szC = C * LDC * 2;
    static constexpr int oKr = 0;                     // K e^{G - G_start(blk)}, then K e^G
    static constexpr int oQr = oKr + szK;             // Q e^{G - G_start(blk)}, then Q e^G
    static constexpr int oKc = oQr + szK;             // K e^{G_end(blk) - G}, then K e^{G_C - G}
    static constexpr int oAt = oKc + szK;             // A^T
    static constexpr int oTt = oAt + szC;             // T^T
    static constexpr int oNt = oTt + szC;             // off-diagonal blocks of N^T (fp16)
    static constexpr int oXt = oNt + szC;             // X^T, X = N^{-1} (fp16)
    static constexpr int oNd = oXt + szC;             // diagonal blocks of N^T (fp32)
    static constexpr int oGl = oNd + 4 * 16 * LDN * 4;  // block-local cumulative log-decay [C][LDG]
    static constexpr int oVt = oGl + C * LDG * 4;     // V^T fp32 [32][LDV]
    static constexpr int oOt = oVt + 32 * LDV * 4;    // O^T bf16 [32][LDO]
    // per-chunk tables (fp32 natural channel order unless noted)
    static constexpr int oFB = oOt + 32 * LDO * 2;    // beta [C]
    static constexpr int oFDl = oFB + C * 4;          // Delta_b = G_loc(15) of block b [4][DK]
    static constexpr int oFGm = oFDl + 4 * DK * 4;    // G_loc(8) of block b [4][DK]
    static constexpr int oFE = oFGm + 4 * DK * 4;     // e^{G_C} [DK]
    static constexpr int oHD = oFE + DK * 4;          // fp16, permuted order: d-factors [3][DK]
    static constexpr int oHMR = oHD + 3 * DK * 2;     // fp16 permuted: e^{-G_loc(8)} [4][DK]
    static constexpr int oHMC = oHMR + 4 * DK * 2;    // fp16 permuted: e^{G_loc(8) - Delta_b} [4][DK]
    static constexpr int oHP = oHMC + 4 * DK * 2;     // fp16 permuted: e^{G_start(b)} [4][DK]
    static constexpr int oHS = oHP + 4 * DK * 2;      // fp16 permuted: e^{G_C - G_end(b)} [4][DK]
    static constexpr int oFlag = oHS + 4 * DK * 2;    // int [4]: block needs the bf16 diagonal path
    static constexpr int total = oFlag + 16;
    static_assert(total <= 160 * 1024, "LDS budget of one gfx950 CU exceeded");
    static_assert((oAt | oTt | oNt | oXt | oNd | oGl | oVt | oOt | oFB | oFDl | oFGm | oFE | oHD | oHMR | oHMC |
                   oHP | oHS | oFlag) % 16 == 0,
                  "alignment");
};

__device__ __forceinline__ void mma16_bf16(float4v& acc, const bf16x8& a, const bf16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ half8 hmul8(const half8& a, const half8& b) { return a * b; }
__device__ __forceinline__ uint2 bld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return uint2{v[0], v[1]};
}

template <int DK>
__global__ __launch_bounds__(256, 1) void chunk_kda_kernel(const KdaArgs a) {
    using L = KdaLds<DK>;
    constexpr int C = kChunk;
    constexpr int NKB = DK / 32;
    constexpr int NST = DK / 16;
    constexpr int KVL = C * DK / 8 / 256;  // 16-byte vectors of one K chunk per lane
    constexpr int CPL = DK / 64;           // channels per lane in the scan
    extern __shared__ __attribute__((aligned(16))) char smem[];
    _Float16* Kr = reinterpret_cast<_Float16*>(smem + L::oKr);
    _Float16* Qr = reinterpret_cast<_Float16*>(smem + L::oQr);
    _Float16* Kc = reinterpret_cast<_Float16*>(smem + L::oKc);
    _Float16* At = reinterpret_cast<_Float16*>(smem + L::oAt);
    _Float16* Tt = reinterpret_cast<_Float16*>(smem + L::oTt);
    _Float16* Nt = reinterpret_cast<_Float16*>(smem + L::oNt);
    _Float16* Xt = reinterpret_cast<_Float16*>(smem + L::oXt);
    float* Nd = reinterpret_cast<float*>(smem + L::oNd);
    float* Gl = reinterpret_cast<float*>(smem + L::oGl);
    float* Vt = reinterpret_cast<float*>(smem + L::oVt);
    _Float16* Ot = reinterpret_cast<_Float16*>(smem + L::oOt);  // bf16 bit patterns
    float* FB = reinterpret_cast<float*>(smem + L::oFB);
    float* FDl = reinterpret_cast<float*>(smem + L::oFDl);
    float* FGm = reinterpret_cast<float*>(smem + L::oFGm);
    float* FE = reinterpret_cast<float*>(smem + L::oFE);
    _Float16* HD = reinterpret_cast<_Float16*>(smem + L::oHD);
    _Float16* HMR = reinterpret_cast<_Float16*>(smem + L::oHMR);
    _Float16* HMC = reinterpret_cast<_Float16*>(smem + L::oHMC);
    _Float16* HP = reinterpret_cast<_Float16*>(smem + L::oHP);
    _Float16* HS = reinterpret_cast<_Float16*>(smem + L::oHS);
    int* Flag = reinterpret_cast<int*>(smem + L::oFlag);

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, j = l & 15, g = l >> 4;
    const int vi = xcd_major_index(blockIdx.x, gridDim.x);
    const int64_t bh = vi / a.ntiles;
    const int dv0 = (vi % a.ntiles) * 32;
    const int64_t T = a.T;
    const int DV = a.dv;
    const auto rq = make_rsrc(a.q + bh * T * DK, (uint32_t)(T * DK * 2));
    const auto rk = make_rsrc(a.k + bh * T * DK, (uint32_t)(T * DK * 2));
    const auto rv = make_rsrc(a.v + bh * T * DV, (uint32_t)(T * DV * 2));
    const auto rg = make_rsrc(a.g + bh * T * DK, (uint32_t)(T * DK * 4));
    const auto rb = make_rsrc(a.beta + bh * T, (uint32_t)(T * 4));
    const auto ro = make_rsrc(a.o + bh * T * DV, (uint32_t)(T * DV * 2));
    const int dvc = dv0 + 16 * w;  // first value channel of consumer wave w (w < 2)
    const int64_t nC = (T + C - 1) / C;

    auto trfrag = [&](const _Float16* base, int ld, int kb, int col) {
        const _Float16* p0 = base + (32 * kb + 4 * g + (j >> 2)) * ld + col;
        return cat8(ldtr(p0), ldtr(p0 + 16 * ld));
    };

    // structural zeros of the triangular operands (never written afterwards)
    for (int i = tid; i < (L::oNd + 4 * 16 * L::LDN * 4 - L::oAt) / 16; i += 256)
        reinterpret_cast<uint4*>(smem + L::oAt)[i] = uint4{0u, 0u, 0u, 0u};

    // ---- state of consumer waves 0-1: S^T tiles (fp32) and their fp16 operand copy
    float4v St[NST];
    half8 Sb[NKB];
#pragma unroll
    for (int t = 0; t < NST; ++t) St[t] = zero4();
    if (w < 2 && a.S0 != nullptr) {
        const float* s0 = a.S0 + bh * (int64_t)DV * DK + (int64_t)(dvc + j) * DK;
#pragma unroll
        for (int t = 0; t < NST; ++t) St[t] = ld4f(s0 + 16 * t + 4 * g);
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) Sb[kb] = pack8(St[2 * kb], St[2 * kb + 1]);

    // ---- prefetch registers for one chunk
    float2 gp[16];  // g of tokens 16w + t, channels CPL*l (+1)
    uint4 kp[KVL], qp[KVL], vp;
    float bp = 0.0f;
    auto issue = [&](int64_t c) {
        const uint32_t t0 = (uint32_t)(c * C);
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const uint32_t off = ((t0 + 16 * w + t) * DK + CPL * l) * 4;
            if constexpr (CPL == 2) {
                const uint2 u = bld8(rg, off);
                gp[t] = float2{__uint_as_float(u.x), __uint_as_float(u.y)};
            } else {
                gp[t] = float2{bld4(rg, off), 0.0f};
            }
        }
#pragma unroll
        for (int u = 0; u < KVL; ++u) {
            const int idx = tid + 256 * u, row = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            const uint32_t off = ((t0 + row) * DK + col) * 2;
            kp[u] = bld16(rk, off);
            qp[u] = bld16(rq, off);
        }
        vp = bld16(rv, ((t0 + (tid >> 2)) * DV + dv0 + (tid & 3) * 8) * 2);
        if (w == 0) bp = bld4(rb, (t0 + l) * 4);
    };

    // Operand fragments (row j of tile ti, reduction block kb) of the Gram products.
    auto rfrag = [&](const _Float16* M, int ti, int kb) { return ld8(M + (16 * ti + j) * L::LDK + 32 * kb + 8 * g); };
    auto hfrag = [&](const _Float16* H, int row, int kb) { return ld8(H + row * DK + 32 * kb + 8 * g); };
    // Diagonal-tile operand of block b built afresh in fp32 from the bf16 input (lane row or
    // column j = token 16b + j; the fragment's channels are 32kb + 4g + e and 32kb + 16 + 4g
    // + e): x e^{G_loc(tok) - G_loc(8)} for the row side, x e^{G_loc(8) - G_loc(tok)} for
    // the column side, rounded to bf16.
    auto diag_bf16 = [&](const __amdgpu_buffer_rsrc_t& rs, int64_t c, int b, int kb, bool row_side) {
        const int tok = 16 * b + j, ch = 32 * kb + 4 * g;
        const uint32_t off = ((uint32_t)(c * C + tok) * DK + ch) * 2;
        const uint2 lo = bld8(rs, off), hi = bld8(rs, off + 32);
        const uint32_t wv[4] = {lo.x, lo.y, hi.x, hi.y};
        const float* gt = Gl + tok * L::LDG + ch;
        const float* gm = Gl + (16 * b + 8) * L::LDG + ch;
        const float4v t0 = ld4f(gt), t1 = ld4f(gt + 16), m0 = ld4f(gm), m1 = ld4f(gm + 16);
        bf16x8 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float d0 = row_side ? t0[e] - m0[e] : m0[e] - t0[e];
            const float d1 = row_side ? t1[e] - m1[e] : m1[e] - t1[e];
            const float x0 = __uint_as_float(e & 1 ? (wv[e >> 1] & 0xffff0000u) : (wv[e >> 1] << 16));
            const float x1 = __uint_as_float(e & 1 ? (wv[2 + (e >> 1)] & 0xffff0000u) : (wv[2 + (e >> 1)] << 16));
            r[e] = (__bf16)(x0 * fast_exp(d0));
            r[4 + e] = (__bf16)(x1 * fast_exp(d1));
        }
        return r;
    };

    lds_barrier();
    if (nC > 0) issue(0);

    for (int64_t c = 0; c < nC; ++c) {
        // ================= S1: block-local scan of the log-decay; V and beta =================
        {
            float G[16][CPL];
            float run[CPL];
#pragma unroll
            for (int e = 0; e < CPL; ++e) run[e] = 0.0f;
            bool unsafe = false;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const float gv[2] = {gp[t].x, gp[t].y};
#pragma unroll
                for (int e = 0; e < CPL; ++e) {
                    run[e] += gv[e];
                    G[t][e] = run[e];
                }
            }
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                const float gm = G[8][e];
                unsafe |= fabsf(gm) > 6.0f;  // the block start, G_loc = 0
#pragma unroll
                for (int t = 0; t < 16; ++t) unsafe |= fabsf(G[t][e] - gm) > 6.0f;
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                float* dst = Gl + (16 * w + t) * L::LDG + CPL * l;
                if constexpr (CPL == 2) *reinterpret_cast<float2*>(dst) = float2{G[t][0], G[t][1]};
                else dst[0] = G[t][0];
            }
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                FDl[w * DK + CPL * l + e] = G[15][e];
                FGm[w * DK + CPL * l + e] = G[8][e];
            }
            const bool any_unsafe = __any(unsafe);
            if (l == 0) Flag[w] = any_unsafe ? 1 : 0;
            if (w == 0) FB[l] = bp;
            // V^T tile, fp32 [channel][token]
            const int row = tid >> 2, col = (tid & 3) * 8;
            const uint32_t ww[4] = {vp.x, vp.y, vp.z, vp.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Vt[(col + 2 * e) * L::LDV + row] = __uint_as_float(ww[e] << 16);
                Vt[(col + 2 * e + 1) * L::LDV + row] = __uint_as_float(ww[e] & 0xffff0000u);
            }
        }
        lds_barrier();

        // ================= S2: per-channel tables; scaled operand copies =================
        if (tid < DK) {
            const int ch = tid, pc = pperm(ch);
            float D[4], Gm[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                D[b] = FDl[b * DK + ch];
                Gm[b] = FGm[b * DK + ch];
            }
            const float P[4] = {0.0f, D[0], D[0] + D[1], D[0] + D[1] + D[2]};
            const float GC = P[3] + D[3];
            FE[ch] = fast_exp(GC);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                HMR[b * DK + pc] = (_Float16)fast_exp(-Gm[b]);
                HMC[b * DK + pc] = (_Float16)fast_exp(Gm[b] - D[b]);
                HP[b * DK + pc] = (_Float16)fast_exp(P[b]);
                HS[b * DK + pc] = (_Float16)fast_exp(GC - P[b] - D[b]);
            }
            // column factors of the tiles two or three blocks below the diagonal:
            // (2,0): e^{Delta_1}, (3,1): e^{Delta_2}, (3,0): e^{Delta_1 + Delta_2}
            HD[0 * DK + pc] = (_Float16)fast_exp(D[1]);
            HD[1 * DK + pc] = (_Float16)fast_exp(D[2]);
            HD[2 * DK + pc] = (_Float16)fast_exp(D[1] + D[2]);
        }
#pragma unroll
        for (int u = 0; u < KVL; ++u) {
            const int idx = tid + 256 * u, row = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            const float* gr = Gl + row * L::LDG + col;
            const float* dl = FDl + (row >> 4) * DK + col;
            const float4v g0 = ld4f(gr), g1 = ld4f(gr + 4), d0 = ld4f(dl), d1 = ld4f(dl + 4);
            float er[8], ec[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                er[e] = fast_exp(g0[e]);
                er[4 + e] = fast_exp(g1[e]);
                ec[e] = fast_exp(d0[e] - g0[e]);
                ec[4 + e] = fast_exp(d1[e] - g1[e]);
            }
            const uint32_t kw[4] = {kp[u].x, kp[u].y, kp[u].z, kp[u].w};
            const uint32_t qw[4] = {qp[u].x, qp[u].y, qp[u].z, qp[u].w};
            half4 kr0, kr1, qr0, qr1, kc0, kc1;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float k0 = __uint_as_float(kw[e] << 16), k1 = __uint_as_float(kw[e] & 0xffff0000u);
                const float k2 = __uint_as_float(kw[2 + e] << 16), k3 = __uint_as_float(kw[2 + e] & 0xffff0000u);
                const float q0 = __uint_as_float(qw[e] << 16), q1 = __uint_as_float(qw[e] & 0xffff0000u);
                const float q2 = __uint_as_float(qw[2 + e] << 16), q3 = __uint_as_float(qw[2 + e] & 0xffff0000u);
                kr0[2 * e] = (_Float16)(k0 * er[2 * e]);
                kr0[2 * e + 1] = (_Float16)(k1 * er[2 * e + 1]);
                kr1[2 * e] = (_Float16)(k2 * er[4 + 2 * e]);
                kr1[2 * e + 1] = (_Float16)(k3 * er[4 + 2 * e + 1]);
                qr0[2 * e] = (_Float16)(q0 * er[2 * e]);
                qr0[2 * e + 1] = (_Float16)(q1 * er[2 * e + 1]);
                qr1[2 * e] = (_Float16)(q2 * er[4 + 2 * e]);
                qr1[2 * e + 1] = (_Float16)(q3 * er[4 + 2 * e + 1]);
                kc0[2 * e] = (_Float16)(k0 * ec[2 * e]);
                kc0[2 * e + 1] = (_Float16)(k1 * ec[2 * e + 1]);
                kc1[2 * e] = (_Float16)(k2 * ec[4 + 2 * e]);
                kc1[2 * e + 1] = (_Float16)(k3 * ec[4 + 2 * e + 1]);
            }
            const int p0 = row * L::LDK + pperm(col), p1 = row * L::LDK + pperm(col + 4);
            *reinterpret_cast<half4*>(Kr + p0) = kr0;
            *reinterpret_cast<half4*>(Kr + p1) = kr1;
            *reinterpret_cast<half4*>(Qr + p0) = qr0;
            *reinterpret_cast<half4*>(Qr + p1) = qr1;
            *reinterpret_cast<half4*>(Kc + p0) = kc0;
            *reinterpret_cast<half4*>(Kc + p1) = kc1;
        }
        // the next chunk's loads fly during the rest of this one
        if (c + 1 < nC) issue(c + 1);
        lds_barrier();

        // ================= S3: Gram tiles =================
        // waves 0-1: K rows (N), waves 2-3: Q rows (A); half 0 tiles {00,10,11,20,30}, half 1
        // {21,22,31,32,33}.  Column factor code: -1 none, 0..2 d-factor pair, 3 diagonal.
        {
            const bool isQ = w >= 2;
            const int h = w & 1;
            const _Float16* Rs = isQ ? Qr : Kr;
            constexpr int NT = 5;
            const int ti_[2][NT] = {{0, 1, 1, 2, 3}, {2, 2, 3, 3, 3}};
            const int tj_[2][NT] = {{0, 0, 1, 0, 0}, {1, 2, 1, 2, 3}};
            const int cf_[2][NT] = {{3, -1, 3, 0, 2}, {-1, 3, 1, -1, 3}};
            float4v acc[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] = zero4();
            int fl[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) fl[b] = Flag[b];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const int ti = ti_[h][t], tj = tj_[h][t], cf = cf_[h][t];
                    half8 A = rfrag(Rs, ti, kb), B = rfrag(Kc, tj, kb);
                    if (cf == 3) {
                        const int b = ti;
                        if (fl[b]) {
                            mma16_bf16(acc[t], diag_bf16(isQ ? rq : rk, c, b, kb, true), diag_bf16(rk, c, b, kb, false));
                        } else {
                            mma16(acc[t], hmul8(A, hfrag(HMR, b, kb)), hmul8(B, hfrag(HMC, b, kb)));
                        }
                    } else {
                        if (cf >= 0) B = hmul8(B, hfrag(HD, cf, kb));
                        mma16(acc[t], A, B);
                    }
                }
            }
            // epilogue: beta of the row for N, causal masks on the diagonal
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int ti = ti_[h][t], tj = tj_[h][t];
                const int m = 16 * tj + j, l0 = 16 * ti + 4 * g;
                float v[4];
                if (!isQ) {
                    const float4v bl = ld4f(FB + l0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = acc[t][r] * bl[r];
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = acc[t][r];
                }
                if (ti == tj) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int lr = l0 + r;
                        if (isQ) v[r] = (m <= lr) ? v[r] : 0.0f;
                        else v[r] = (m < lr) ? v[r] : (m == lr ? 1.0f : 0.0f);
                    }
                }
                if (ti == tj && !isQ) {
                    *reinterpret_cast<float4v*>(Nd + (ti * 16 + j) * L::LDN + 4 * g) = float4v{v[0], v[1], v[2], v[3]};
                } else {
                    _Float16* dst = (isQ ? At : Nt) + m * L::LDC + l0;
                    *reinterpret_cast<half4*>(dst) = half4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
                }
            }
        }
        lds_barrier();

        // ================= S4: diagonal inverses (block w per wave) =================
        float xd[16];
        {
            const int b = w, jc = j;
            const float* nb = Nd + b * 16 * L::LDN;
            float4v nr[15][4];
#pragma unroll
            for (int i = 0; i < 15; ++i)
#pragma unroll
                for (int q4 = (i + 1) / 4; q4 < 4; ++q4) nr[i][q4] = ld4f(nb + i * L::LDN + 4 * q4);
#pragma unroll
            for (int t = 0; t < 16; ++t) xd[t] = (t == jc) ? 1.0f : 0.0f;
#pragma unroll
            for (int i = 0; i < 15; ++i) {
#pragma unroll
                for (int q4 = (i + 1) / 4; q4 < 4; ++q4) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * q4 + e > i) xd[4 * q4 + e] -= nr[i][q4][e] * xd[i];
                }
            }
            if (l < 16) {
                half8 h0, h1;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    h0[t] = (_Float16)xd[t];
                    h1[t] = (_Float16)xd[8 + t];
                }
                *reinterpret_cast<half8*>(Xt + (16 * b + jc) * L::LDC + 16 * b) = h0;
                *reinterpret_cast<half8*>(Xt + (16 * b + jc) * L::LDC + 16 * b + 8) = h1;
            }
        }
        lds_barrier();

        // ================= S5: first block level (waves 0-1); rescale the copies (2-3) ======
        float4v x2 = zero4();
        if (w < 2) {
            const int p = w, b0 = 2 * p, b1 = 2 * p + 1;
            const half4 z4 = {(_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f};
            const half8 fa = cat8(ldtr(Nt + (16 * b0 + 4 * g + (j >> 2)) * L::LDC + 16 * b1 + 4 * (j & 3)), z4);
            const half8 fb = cat8(*reinterpret_cast<const half4*>(Xt + (16 * b0 + j) * L::LDC + 16 * b0 + 4 * g), z4);
            float4v y = zero4();
            mma16(y, fa, fb);
            const half8 fx = cat8(ldtr(Xt + (16 * b1 + 4 * g + (j >> 2)) * L::LDC + 16 * b1 + 4 * (j & 3)), z4);
            const half8 fy = cat8(half4{(_Float16)y[0], (_Float16)y[1], (_Float16)y[2], (_Float16)y[3]}, z4);
            mma16(x2, fx, fy);
#pragma unroll
            for (int r = 0; r < 4; ++r) x2[r] = -x2[r];
            *reinterpret_cast<half4*>(Xt + (16 * b0 + j) * L::LDC + 16 * b1 + 4 * g) =
                half4{(_Float16)x2[0], (_Float16)x2[1], (_Float16)x2[2], (_Float16)x2[3]};
        } else {
            // Kr -> K e^G, Qr -> Q e^G (factor e^{G_start(blk)}), Kc -> K e^{G_C - G}
            // (factor e^{G_C - G_end(blk)}); 16-byte groups of the permuted rows.
            constexpr int NG = C * (DK / 8);  // 16-byte groups per copy
            for (int i = tid - 128; i < NG; i += 128) {
                const int row = i / (DK / 8), col = (i % (DK / 8)) * 8, blk = row >> 4;
                const half8 fp = ld8(HP + blk * DK + col), fs = ld8(HS + blk * DK + col);
                half8* pk = reinterpret_cast<half8*>(Kr + row * L::LDK + col);
                half8* pq = reinterpret_cast<half8*>(Qr + row * L::LDK + col);
                half8* pc = reinterpret_cast<half8*>(Kc + row * L::LDK + col);
                *pk = hmul8(*pk, fp);
                *pq = hmul8(*pq, fp);
                *pc = hmul8(*pc, fs);
            }
        }
        lds_barrier();

        // ================= S6: second block level (waves 0-1) =================
        float4v xc[2] = {zero4(), zero4()};
        if (w < 2) {
            const int p = w, n = 16 * p + j;
            const half8 fxa = cat8(*reinterpret_cast<const half4*>(Xt + n * L::LDC + 4 * g),
                                   *reinterpret_cast<const half4*>(Xt + n * L::LDC + 16 + 4 * g));
            float4v y3[2];
#pragma unroll
            for (int ti = 0; ti < 2; ++ti) {
                y3[ti] = zero4();
                mma16(y3[ti], trfrag(Nt, L::LDC, 0, 32 + 16 * ti + 4 * (j & 3)), fxa);
            }
            const half8 fy = pack8(y3[0], y3[1]);
#pragma unroll
            for (int ti = 0; ti < 2; ++ti) {
                mma16(xc[ti], trfrag(Xt, L::LDC, 1, 32 + 16 * ti + 4 * (j & 3)), fy);
#pragma unroll
                for (int r = 0; r < 4; ++r) xc[ti][r] = -xc[ti][r];
            }
        }
        lds_barrier();

        // ================= S7: T = X diag(beta), column-major =================
        {
            const int b = w;
            if (l < 16) {
                const int m = 16 * b + j;
                const float bm = FB[m];
                half8 h0, h1;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    h0[t] = (_Float16)(xd[t] * bm);
                    h1[t] = (_Float16)(xd[8 + t] * bm);
                }
                *reinterpret_cast<half8*>(Tt + m * L::LDC + 16 * b) = h0;
                *reinterpret_cast<half8*>(Tt + m * L::LDC + 16 * b + 8) = h1;
            }
            if (w < 2) {
                const int p = w;
                {
                    const int m = 32 * p + j;
                    const float bm = FB[m];
                    *reinterpret_cast<half4*>(Tt + m * L::LDC + 32 * p + 16 + 4 * g) =
                        half4{(_Float16)(x2[0] * bm), (_Float16)(x2[1] * bm), (_Float16)(x2[2] * bm), (_Float16)(x2[3] * bm)};
                }
                {
                    const int m = 16 * p + j;
                    const float bm = FB[m];
#pragma unroll
                    for (int ti = 0; ti < 2; ++ti)
                        *reinterpret_cast<half4*>(Tt + m * L::LDC + 32 + 16 * ti + 4 * g) =
                            half4{(_Float16)(xc[ti][0] * bm), (_Float16)(xc[ti][1] * bm), (_Float16)(xc[ti][2] * bm),
                                  (_Float16)(xc[ti][3] * bm)};
                }
            }
        }
        lds_barrier();

        // ================= S8: state pass of chunk c (waves 0-1) =================
        if (w < 2) {
            // P_K = (K e^G) S^T, P_Q = (Q e^G) S^T
            float4v PK[4], PQ[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                PK[ti] = zero4();
                PQ[ti] = zero4();
            }
            half8 fa[8], fb[8];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                fa[ti] = rfrag(Kr, ti, 0);
                fa[4 + ti] = rfrag(Qr, ti, 0);
            }
            float4v vv[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) vv[ti] = ld4f(Vt + (16 * w + j) * L::LDV + 16 * ti + 4 * g);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                half8* cur = (kb & 1) ? fb : fa;
                half8* nxt = (kb & 1) ? fa : fb;
                if (kb + 1 < NKB) {
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti) {
                        nxt[ti] = rfrag(Kr, ti, kb + 1);
                        nxt[4 + ti] = rfrag(Qr, ti, kb + 1);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
                    mma16(PK[ti], cur[ti], Sb[kb]);
                    mma16(PQ[ti], cur[4 + ti], Sb[kb]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            half8 tf[6], af[6];
#pragma unroll
            for (int ti = 0, n = 0; ti < 4; ++ti) {
#pragma unroll
                for (int kb = 0; kb <= (ti >> 1); ++kb, ++n) {
                    tf[n] = trfrag(Tt, L::LDC, kb, 16 * ti + 4 * (j & 3));
                    af[n] = trfrag(At, L::LDC, kb, 16 * ti + 4 * (j & 3));
                }
            }
            float4v ed[NST];
#pragma unroll
            for (int t = 0; t < NST; ++t) ed[t] = ld4f(FE + 16 * t + 4 * g);
            __builtin_amdgcn_sched_barrier(0);
            float4v Rr[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int r = 0; r < 4; ++r) Rr[ti][r] = vv[ti][r] - PK[ti][r];
            const half8 rB[2] = {pack8(Rr[0], Rr[1]), pack8(Rr[2], Rr[3])};
            float4v Zz[4];
#pragma unroll
            for (int ti = 0, n = 0; ti < 4; ++ti) {
                Zz[ti] = zero4();
#pragma unroll
                for (int kb = 0; kb <= (ti >> 1); ++kb, ++n) mma16(Zz[ti], tf[n], rB[kb]);
            }
            auto ktfrag = [&](int t, int kb) { return trfrag(Kc, L::LDK, kb, pperm(16 * t + 4 * (j & 3))); };
            half8 kt0[NST], kt1[NST];
#pragma unroll
            for (int t = 0; t < NST; ++t) {
                kt0[t] = ktfrag(t, 0);
                kt1[t] = ktfrag(t, 1);
            }
            const half8 zB[2] = {pack8(Zz[0], Zz[1]), pack8(Zz[2], Zz[3])};
#pragma unroll
            for (int ti = 0, n = 0; ti < 4; ++ti) {
                float4v acc = PQ[ti];
#pragma unroll
                for (int kb = 0; kb <= (ti >> 1); ++kb, ++n) mma16(acc, af[n], zB[kb]);
                *reinterpret_cast<uint2*>(Ot + (16 * w + j) * L::LDO + 16 * ti + 4 * g) =
                    uint2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
            }
            lds_fence();
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int tb = 32 * s2 + 16 * (g >> 1), d = 16 * w + 8 * (g & 1);
                const _Float16* rp = Ot + (d + (j >> 2)) * L::LDO + tb + 4 * (j & 3);
                const uint2 lo = __builtin_bit_cast(uint2, ldtr(rp));
                const uint2 hi = __builtin_bit_cast(uint2, ldtr(rp + 4 * L::LDO));
                bst16(ro, ((uint32_t)(c * C + tb + j) * DV + dv0 + d) * 2, uint4{lo.x, lo.y, hi.x, hi.y});
            }
            // S^T <- Diag(e^{G_C}) S^T + (K e^{G_C - G})^T Z
#pragma unroll
            for (int t = 0; t < NST; ++t) {
#pragma unroll
                for (int r = 0; r < 4; ++r) St[t][r] *= ed[t][r];
                mma16(St[t], kt0[t], zB[0]);
                mma16(St[t], kt1[t], zB[1]);
            }
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) Sb[kb] = pack8(St[2 * kb], St[2 * kb + 1]);
        }
        lds_barrier();
    }

    if (w < 2 && a.Sf != nullptr) {
        float* sf = a.Sf + bh * (int64_t)DV * DK + (int64_t)(dvc + j) * DK;
#pragma unroll
        for (int t = 0; t < NST; ++t) *reinterpret_cast<float4v*>(sf + 16 * t + 4 * g) = St[t];
    }
}

template <int DK>
static hipError_t launch_kda(const KdaArgs& a, int64_t nwg, hipStream_t st) {
    using L = KdaLds<DK>;
    auto kern = chunk_kda_kernel<DK>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, L::total);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(256), L::total, st, a);
    return hipGetLastError();
}

hipError_t chunk_kda_dispatch(int64_t BH, int64_t T, int dk, int dv, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, const float* S0, void* o, float* Sf,
                              hipStream_t st) {
    KdaArgs a;
    a.T = T;
    a.dv = dv;
    a.ntiles = dv / 32;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.g = g;
    a.beta = beta;
    a.S0 = S0;
    a.o = static_cast<uint16_t*>(o);
    a.Sf = Sf;
    const int64_t nwg = BH * a.ntiles;
    if (dk == 128) return launch_kda<128>(a, nwg, st);
    return launch_kda<64>(a, nwg, st);
}

}  // namespace gdr
