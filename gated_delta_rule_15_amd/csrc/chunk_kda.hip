// chunk_kda.hip -- UT pass of the chunked forward with a per-channel gate (KDA-style) and of
// Gated DeltaNet-2, bf16 inputs, fp16 MFMA operands, fp32 accumulation, gfx950.  The state
// pass that follows it is chunk_state_kernel (chunk_split.hip) in its per-channel modes.
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
// Everything but the last three lines depends on the chunk alone; this kernel forms it for all
// chunks at once.  The decay sits inside the channel sum, so the Gram products take it on their
// operands:
//   off-diagonal 16x16 tiles (row block bi > column block bj), reference = end of block bj:
//     row operand  K_l e^{G_l - G_start(bi)}            ("Kr", <= 1, one copy of K and Q)
//     column       K_m e^{G_end(bj) - G_m}              ("Kc", <= 1)
//     times the per-channel factor e^{G_start(bi) - G_end(bj)} (<= 1) on the column fragment;
//   diagonal tiles, reference = token 8 of the block: Kr and Kc times e^{-G_loc(8)} and
//     e^{G_loc(8) - G_loc(15)}, per channel (G_loc = cumulative log-decay from the block
//     start).  Those factors exceed 1 by up to e^{8|g|}.  While every |G_loc(t) - G_loc(8)|
//     (t = -1..15, G_loc(-1) = 0) stays within 6 the fp16 path is exact to fp16 rounding.
//     A block beyond that ("flagged") is formed afresh from the bf16 inputs with every factor
//     of the form e^{G_i - G_j}, i >= j, so at most 1 whatever the decay (see diag_exact).
//
// One workgroup (four waves) per (sequence, run of consecutive chunks), all runs at once; each
// chunk runs stage by stage with all waves: scan, staging, Gram, the inverses of the four 16x16
// diagonal blocks of N, the blocks of N^{-1} below the diagonal
// (M_bc = -X_bb sum_{c<=d<b} N_bd M_dc), and the copy-out.  Loads of the next chunk are in
// flight while a chunk is processed.  Per (sequence, chunk) the workspace receives the operands
// of the state pass: A^T and T = N^{-1} diag(beta) (fp16, T's columns pperm'd), the decayed
// copies K e^G, Q e^G and K e^{G_C - G} (fp16, rescaled on the way out) and e^{G_C} per key
// channel (fp32).  Waves 2-3 write the copies while waves 0-1 form the inverses.
//
// Gated DeltaNet-2 ("Gated DeltaNet-2, and the gate that was doing two jobs", section 2) is
// the GD2 instantiation.  The scalar beta is replaced by a key-side erase gate b_t and a
// value-side write gate w_t: S_t = S_{t-1} D_t (I - e_t k_t^T) + z_t k_t^T, with e = b (.) k
// and z = w (.) v.  Per chunk, the same derivation gives
//   L[l][m] = sum_c e_lc k_mc e^{G_lc - G_mc} (m < l),   N = I + L,   Z = N^{-1} R,
//   R = Z_in - (E (.) e^G) S^T   (Z_in the rows z_l),
// and O, A and the state update unchanged: only the row operand of N and of the prediction
// product changes from beta k to e, and the right-hand side from beta v to z (formed by the
// state pass).  So the "Kr" copy holds E e^{G - G_start(blk)} (then E e^G), and beta is not used.
#include <type_traits>

#include "chunk_common.h"

namespace gdr {

struct KdaArgs {
    int64_t T;
    const uint16_t* q;
    const uint16_t* k;
    const float* g;  // [.., T, DK]
    const float* beta;
    const float* eg;  // erase gate b [.., T, DK] (GD2)
    uint16_t* ws;     // kda_ws_stride<DK>() halfs per (sequence, chunk)
    int cpw;          // chunks per workgroup
};

template <int DK>
struct KdaLds {
    static constexpr int C = kChunk;
    static constexpr int LDK = DK + 16;  // halfs, rows of the K / Q operand copies (bank-conflict
                                         // free for fragment and transposing reads)
    static constexpr int LDX = 16 + 8;   // halfs, rows of a 16x16 fp16 block
    static constexpr int LDC = C + 8;    // halfs, rows of C-wide fp16 matrices
    static constexpr int LDN = 16 + 4;   // floats, rows of a 16x16 fp32 block
    static constexpr int LDG = DK + 4;   // floats, rows of the block-local cumulative log-decay
    static constexpr int szK = C * LDK * 2;
    static constexpr int szC = C * LDC * 2;
    // The per-chunk tables come first: the Gram stage reads them every few instructions, and
    // below 64 KiB an LDS address folds into the instruction's 16-bit offset instead of taking
    // a register of its own.  Tables are fp32 in natural channel order unless noted.
    static constexpr int oFB = 0;                     // beta [C]
    static constexpr int oFDl = oFB + C * 4;          // Delta_b = G_loc(15) of block b [4][DK]
    static constexpr int oFE = oFDl + 4 * DK * 4;     // e^{G_C} [DK]
    static constexpr int oHD = oFE + DK * 4;          // fp16: d-factors [3][DK]
    static constexpr int oHMR = oHD + 3 * DK * 2;     // fp16: e^{-G_loc(8)} [4][DK]
    static constexpr int oHMC = oHMR + 4 * DK * 2;    // fp16: e^{G_loc(8) - Delta_b} [4][DK]
    static constexpr int oHP = oHMC + 4 * DK * 2;     // fp16: e^{G_start(b)} [4][DK]
    static constexpr int oHS = oHP + 4 * DK * 2;      // fp16: e^{G_C - G_end(b)} [4][DK]
    static constexpr int oFlag = oHS + 4 * DK * 2;    // int [4]: block takes the exact diagonal path
    static constexpr int oKr = oFlag + 16;            // K e^{G - G_start(blk)}
    static constexpr int oQr = oKr + szK;             // Q e^{G - G_start(blk)}
    static constexpr int oKc = oQr + szK;             // K e^{G_end(blk) - G}
    static constexpr int oAt = oKc + szK;             // A^T
    static constexpr int oNt = oAt + szC;             // off-diagonal blocks of N^T (fp16)
    static constexpr int oXd = oNt + szC;             // X_bb^T, diagonal blocks of N^{-1} (fp16)
    static constexpr int oNd = oXd + 4 * 16 * LDX * 2;  // diagonal blocks of N^T (fp32)
    static constexpr int oGl = oNd + 4 * 16 * LDN * 4;  // block-local cumulative log-decay [C][LDG]
    static constexpr int oTt = oGl + C * LDG * 4;     // T, staged for the copy-out
    static constexpr int total = oTt + szC;
    static_assert(total <= 160 * 1024, "LDS budget of one gfx950 CU exceeded");
    static_assert((oKr | oAt | oNt | oXd | oNd | oGl | oTt | oFDl | oFE | oHD | oHMR | oHMC |
                   oHP | oHS | oFlag) % 16 == 0,
                  "alignment");
};

__device__ __forceinline__ half8 hmul8(const half8& a, const half8& b) { return a * b; }
__device__ __forceinline__ uint2 bld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return uint2{v[0], v[1]};
}

template <int DK, bool GD2>
__global__ __launch_bounds__(256, 1) void chunk_kda_kernel(const KdaArgs a) {
    using L = KdaLds<DK>;
    constexpr int C = kChunk;
    constexpr int NKB = DK / 32;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    _Float16* Kr = reinterpret_cast<_Float16*>(smem + L::oKr);
    _Float16* Qr = reinterpret_cast<_Float16*>(smem + L::oQr);
    _Float16* Kc = reinterpret_cast<_Float16*>(smem + L::oKc);
    _Float16* At = reinterpret_cast<_Float16*>(smem + L::oAt);
    _Float16* Nt = reinterpret_cast<_Float16*>(smem + L::oNt);
    _Float16* Xd = reinterpret_cast<_Float16*>(smem + L::oXd);
    _Float16* Tt = reinterpret_cast<_Float16*>(smem + L::oTt);
    float* Nd = reinterpret_cast<float*>(smem + L::oNd);
    float* Gl = reinterpret_cast<float*>(smem + L::oGl);
    float* FB = reinterpret_cast<float*>(smem + L::oFB);
    float* FDl = reinterpret_cast<float*>(smem + L::oFDl);
    float* FE = reinterpret_cast<float*>(smem + L::oFE);
    _Float16* HD = reinterpret_cast<_Float16*>(smem + L::oHD);
    _Float16* HMR = reinterpret_cast<_Float16*>(smem + L::oHMR);
    _Float16* HMC = reinterpret_cast<_Float16*>(smem + L::oHMC);
    _Float16* HP = reinterpret_cast<_Float16*>(smem + L::oHP);
    _Float16* HS = reinterpret_cast<_Float16*>(smem + L::oHS);
    int* Flag = reinterpret_cast<int*>(smem + L::oFlag);

    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, j = l & 15, g = l >> 4;
    const int64_t T = a.T;
    const int64_t nC = (T + C - 1) / C;
    // one group per (sequence, run of cpw consecutive chunks)
    const int64_t runs = (nC + a.cpw - 1) / a.cpw;
    const int64_t bh = blockIdx.x / runs;
    const int64_t c_first = (blockIdx.x - bh * runs) * a.cpw;
    const int64_t c_last = c_first + a.cpw < nC ? c_first + a.cpw : nC;
    const auto rq = make_rsrc(a.q + bh * T * DK, (uint32_t)(T * DK * 2));
    const auto rk = make_rsrc(a.k + bh * T * DK, (uint32_t)(T * DK * 2));
    const auto rg = make_rsrc(a.g + bh * T * DK, (uint32_t)(T * DK * 4));
    const auto rb = make_rsrc(GD2 ? nullptr : a.beta + bh * T, GD2 ? 0u : (uint32_t)(T * 4));
    const auto re = make_rsrc(GD2 ? a.eg + bh * T * DK : nullptr, GD2 ? (uint32_t)(T * DK * 4) : 0u);

    // structural zeros of the triangular operands (never written afterwards)
    for (int i = tid; i < (L::oGl - L::oAt) / 16; i += 256)
        reinterpret_cast<uint4*>(smem + L::oAt)[i] = uint4{0u, 0u, 0u, 0u};

    // ---- prefetch registers for one chunk, in the layout of the scan: wave w holds the
    // 16-token block w, lane l the channel pair ch2 = 2 (l mod DK/2) (for DK = 64 the upper
    // half of the wave loads duplicates and stores nothing)
    const int ch2 = 2 * (l % (DK / 2));
    const bool own = 2 * l < DK;
    float2 gp[16], ep[16];  // ep: erase gate b (GD2)
    uint32_t kp[16], qp[16];
    float bp = 0.0f;
    // token t of the lane's block (g, k, q of its channel pair); t = 0 also brings beta.
    // Past the sequence end the loads return zeros (identity tokens).
    // The token's element offset is formed as a wave-uniform value the compiler cannot split, so
    // the address is one add to the lane's channel offset, not one of 16 registers held
    // through the loop.
    auto issue_tok = [&](int64_t c, int t) {
        uint32_t tb = ((uint32_t)(c * C) + 16 * w + t) * DK;
        asm volatile("" : "+s"(tb));
        const uint32_t e = tb + ch2;
        const uint2 u = bld8(rg, e * 4);
        gp[t] = float2{__uint_as_float(u.x), __uint_as_float(u.y)};
        kp[t] = __builtin_amdgcn_raw_buffer_load_b32(rk, e * 2, 0, 0);
        qp[t] = __builtin_amdgcn_raw_buffer_load_b32(rq, e * 2, 0, 0);
        if constexpr (GD2) {
            const uint2 ue = bld8(re, e * 4);
            ep[t] = float2{__uint_as_float(ue.x), __uint_as_float(ue.y)};
        } else if (t == 0) {
            bp = bld4(rb, ((uint32_t)(c * C) + l) * 4);  // every wave: a load under a branch costs a full wait
        }
    };
    auto issue = [&](int64_t c) {
#pragma unroll
        for (int t = 0; t < 16; ++t) issue_tok(c, t);
    };

    // Operand fragments (row j of tile ti, reduction block kb) of the Gram products.
    auto rfrag = [&](const _Float16* M, int ti, int kb) { return ld8(M + (16 * ti + j) * L::LDK + 32 * kb + 8 * g); };
    auto hfrag = [&](const _Float16* H, int row, int kb) { return ld8(H + row * DK + 32 * kb + 8 * g); };

    // Diagonal 16x16 tile of block b of a flagged block, formed without any factor above 1:
    // entry (l, m) = sum_c x_lc k_mc e^{G_lc - G_mc} (x = q, k, or e = b (.) k with `gate`).
    // For l != m let h be the highest bit in which the block-local indices l' and m' differ; for
    // m' < l' the reference token r = l' with the bits below h cleared satisfies m' < r <= l',
    // so e^{G_l - G_m} = e^{G_l - G_r} e^{G_r - G_m} with both factors <= 1 for a decaying gate.
    // Level h multiplies the row operand x_l e^{G_l - G_r(l')} (rows with bit h set, others 0) by
    // the column operand k_m e^{G_r(m') - G_m} (columns with bit h clear, r(m') = m' with bit h
    // set and the bits below cleared); its entries are right exactly where h is the highest
    // differing bit, and each entry takes its value from that level (the diagonal from an
    // unscaled product).  Five fp16 products per reduction block instead of one; only blocks
    // whose in-block decay spread exceeds the fp16 path's range come here.
    auto diag_exact = [&](const __amdgpu_buffer_rsrc_t& rs, int64_t c, int b, bool gate) {
        const int tok = 16 * b + j;
        float4v out = zero4();
        // level 4 is the unscaled product that supplies the diagonal; levels and reduction
        // blocks stay rolled loops, so this rare path keeps few registers live
#pragma nounroll
        for (int lev = 0; lev < 5; ++lev) {
            const bool rowlive = lev == 4 || ((j >> lev) & 1), collive = lev == 4 || !((j >> lev) & 1);
            const int rr = lev == 4 ? tok : 16 * b + ((j >> lev) << lev);        // row reference token
            const int rc = lev == 4 ? tok : 16 * b + (((j >> lev) | 1) << lev);  // column reference token
            float4v acc = zero4();
#pragma nounroll
            for (int kb = 0; kb < NKB; ++kb) {
                const int ch = 32 * kb + 8 * g;
                const uint32_t gidx = (uint32_t)(c * C + tok) * DK + ch;
                const uint4 ur = bld16(rs, gidx * 2), uk = bld16(rk, gidx * 2);
                const uint32_t xr[4] = {ur.x, ur.y, ur.z, ur.w}, xk[4] = {uk.x, uk.y, uk.z, uk.w};
                float gb[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) gb[e] = 1.0f;
                if (gate) {
                    const uint4 b0 = bld16(re, gidx * 4), b1 = bld16(re, gidx * 4 + 16);
                    const uint32_t bw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) gb[e] = __uint_as_float(bw[e]);
                }
                const float* pt = Gl + tok * L::LDG + ch;
                const float* pr = Gl + rr * L::LDG + ch;
                const float* pc = Gl + rc * L::LDG + ch;
                half8 ra, cb;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = gb[e] * __uint_as_float(e & 1 ? (xr[e >> 1] & 0xffff0000u) : (xr[e >> 1] << 16));
                    const float kv = __uint_as_float(e & 1 ? (xk[e >> 1] & 0xffff0000u) : (xk[e >> 1] << 16));
                    ra[e] = rowlive ? (_Float16)(x * fast_exp(pt[e] - pr[e])) : (_Float16)0.0f;
                    cb[e] = collive ? (_Float16)(kv * fast_exp(pc[e] - pt[e])) : (_Float16)0.0f;
                }
                mma16(acc, ra, cb);
            }
            // element (row 4g + r, column j) of the tile takes the level of its highest
            // differing bit
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = (4 * g + r) ^ j;
                const int hb = d == 0 ? 4 : d >= 8 ? 3 : d >= 4 ? 2 : d >= 2 ? 1 : 0;
                out[r] = hb == lev ? acc[r] : out[r];
            }
        }
        return out;
    };

    lds_barrier();
    if (nC > 0) issue(c_first);

    for (int64_t c = c_first; c < c_last; ++c) {
        // ====== S1: block-local scan of the log-decay and the decayed copies of K and Q ======
        // Per channel pair and 16-token block: a_t = e^{g_t}, E_t = e^{G_loc(t)} (forward
        // product), Ec_t = e^{G_loc(15) - G_loc(t)} (backward product);
        // Kr = K E, Qr = Q E, Kc = K Ec.
        {
            float G[16][2], E[16][2], Ec[16][2];
            float run[2] = {0.0f, 0.0f}, pe[2] = {1.0f, 1.0f}, pc[2] = {1.0f, 1.0f};
            float av[16][2];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const float gv[2] = {gp[t].x, gp[t].y};
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    run[e] += gv[e];
                    G[t][e] = run[e];
                    av[t][e] = fast_exp(gv[e]);
                    pe[e] *= av[t][e];
                    E[t][e] = pe[e];
                }
            }
#pragma unroll
            for (int t = 15; t >= 0; --t) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    Ec[t][e] = pc[e];
                    pc[e] *= av[t][e];
                }
            }
            bool unsafe = false;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float gm = G[8][e];
                unsafe |= fabsf(gm) > 6.0f;  // the block start, G_loc = 0
#pragma unroll
                for (int t = 0; t < 16; ++t) unsafe |= fabsf(G[t][e] - gm) > 6.0f;
            }
            if (own) {
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    const int row = 16 * w + t;
                    *reinterpret_cast<float2*>(Gl + row * L::LDG + ch2) = float2{G[t][0], G[t][1]};
                    const float k0 = __uint_as_float(kp[t] << 16), k1 = __uint_as_float(kp[t] & 0xffff0000u);
                    const float q0 = __uint_as_float(qp[t] << 16), q1 = __uint_as_float(qp[t] & 0xffff0000u);
                    // row operand of N and of the prediction: beta k (KDA, beta applied later) or e = b k
                    const float r0 = GD2 ? ep[t].x * k0 : k0, r1 = GD2 ? ep[t].y * k1 : k1;
                    typedef _Float16 half2v __attribute__((ext_vector_type(2)));
                    *reinterpret_cast<half2v*>(Kr + row * L::LDK + ch2) = half2v{(_Float16)(r0 * E[t][0]), (_Float16)(r1 * E[t][1])};
                    *reinterpret_cast<half2v*>(Qr + row * L::LDK + ch2) = half2v{(_Float16)(q0 * E[t][0]), (_Float16)(q1 * E[t][1])};
                    *reinterpret_cast<half2v*>(Kc + row * L::LDK + ch2) = half2v{(_Float16)(k0 * Ec[t][0]), (_Float16)(k1 * Ec[t][1])};
                }
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    FDl[w * DK + ch2 + e] = G[15][e];
                    // diagonal-tile factors of this block: e^{-G_loc(8)}, e^{G_loc(8) - G_loc(15)}
                    HMR[w * DK + ch2 + e] = (_Float16)fast_exp(-G[8][e]);
                    HMC[w * DK + ch2 + e] = (_Float16)fast_exp(G[8][e] - G[15][e]);
                }
            }
            const bool any_unsafe = __any(unsafe);
            if (l == 0) Flag[w] = any_unsafe ? 1 : 0;
            if (!GD2 && w == 0) FB[l] = bp;
        }
        lds_barrier();

        // ================= S2: per-channel tables across the blocks =================
        {
            // spread over all threads: channel tid % DK, a share of the blocks
            const int ch = tid % DK, hb = tid / DK;  // hb in [0, 256 / DK)
            float D[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) D[b] = FDl[b * DK + ch];
            const float P[4] = {0.0f, D[0], D[0] + D[1], D[0] + D[1] + D[2]};
            const float GC = P[3] + D[3];
            constexpr int NH = 256 / DK, BPH = 4 / NH;  // thread groups per channel, blocks each
#pragma unroll
            for (int bb = 0; bb < BPH; ++bb) {
                const int b = hb * BPH + bb;
                HP[b * DK + ch] = (_Float16)fast_exp(P[b]);
                HS[b * DK + ch] = (_Float16)fast_exp(GC - P[b] - D[b]);
            }
            if (hb == 0) {
                FE[ch] = fast_exp(GC);
                // column factors of the tiles two or three blocks below the diagonal:
                // (2,0): e^{Delta_1}, (3,1): e^{Delta_2}, (3,0): e^{Delta_1 + Delta_2}
                HD[0 * DK + ch] = (_Float16)fast_exp(D[1]);
                HD[1 * DK + ch] = (_Float16)fast_exp(D[2]);
                HD[2 * DK + ch] = (_Float16)fast_exp(D[1] + D[2]);
            }
        }
        lds_barrier();

        // ================= S3: Gram tiles =================
        // waves 0-1: K rows (N), waves 2-3: Q rows (A); half 0 tiles {00,10,11,20,30}, half 1
        // {21,22,31,32,33}.  Column factor code: -1 none, 0..2 d-factor pair, 3 diagonal.
        // Each wave runs its own compile-time instance, so every tile's path is static.
        // The next chunk's loads are issued between this stage's MFMAs (a token of the block
        // per step), so the memory queue drains while the matrix pipe works.
        const int64_t cn = c + 1 < c_last ? c + 1 : c;  // reloading the last chunk is harmless
        auto gram_kda = [&](auto hc, auto qc, auto bc) {
            constexpr int h = decltype(hc)::value;
            constexpr bool isQ = decltype(qc)::value;
            constexpr bool BF = decltype(bc)::value;  // some diagonal block of the wave is flagged
            const _Float16* Rs = isQ ? Qr : Kr;
            constexpr int NT = 5;
            constexpr int ti_[2][NT] = {{0, 1, 1, 2, 3}, {2, 2, 3, 3, 3}};
            constexpr int tj_[2][NT] = {{0, 0, 1, 0, 0}, {1, 2, 1, 2, 3}};
            constexpr int cf_[2][NT] = {{3, -1, 3, 0, 2}, {-1, 3, 1, -1, 3}};
            float4v acc[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] = zero4();
            if constexpr (!BF) {
                // every diagonal tile on fp16: the operands of reduction block kb + 1 are read
                // from LDS while the MFMAs of block kb run (two register sets), and their factors
                // applied after them
                half8 oa[2][NT], ob[2][NT], fa[2][NT], fb[2][NT];
                auto read_kb = [&](int kb, half8* ra, half8* rb, half8* ha, half8* hb) {
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const int ti = ti_[h][t], tj = tj_[h][t], cf = cf_[h][t];
                        ra[t] = rfrag(Rs, ti, kb);
                        rb[t] = rfrag(Kc, tj, kb);
                        if (cf == 3) {
                            ha[t] = hfrag(HMR, ti, kb);
                            hb[t] = hfrag(HMC, ti, kb);
                        } else if (cf >= 0) {
                            hb[t] = hfrag(HD, cf, kb);
                        }
                    }
                };
                auto scale_kb = [&](half8* ra, half8* rb, const half8* ha, const half8* hb) {
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const int cf = cf_[h][t];
                        if (cf == 3) ra[t] = hmul8(ra[t], ha[t]);
                        if (cf >= 0) rb[t] = hmul8(rb[t], hb[t]);
                    }
                };
                read_kb(0, oa[0], ob[0], fa[0], fb[0]);
                scale_kb(oa[0], ob[0], fa[0], fb[0]);
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const int cur = kb & 1, nxt = cur ^ 1;
                    if (kb + 1 < NKB) read_kb(kb + 1, oa[nxt], ob[nxt], fa[nxt], fb[nxt]);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        mma16(acc[t], oa[cur][t], ob[cur][t]);
                        if (t < 16 / NKB) issue_tok(cn, kb * (16 / NKB) + t);
                    }
#pragma unroll
                    for (int u = NT; u < 16 / NKB; ++u) issue_tok(cn, kb * (16 / NKB) + u);
                    __builtin_amdgcn_sched_barrier(0);
                    if (kb + 1 < NKB) scale_kb(oa[nxt], ob[nxt], fa[nxt], fb[nxt]);
                }
            } else {
                // flagged diagonal blocks are chosen per block for the whole wave
                int fl[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) fl[b] = __builtin_amdgcn_readfirstlane(Flag[b]);
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const int ti = ti_[h][t], tj = tj_[h][t], cf = cf_[h][t];
                        if (!(cf == 3 && fl[ti])) {
                            half8 A = rfrag(Rs, ti, kb), B = rfrag(Kc, tj, kb);
                            if (cf == 3) {
                                A = hmul8(A, hfrag(HMR, ti, kb));
                                B = hmul8(B, hfrag(HMC, ti, kb));
                            } else if (cf >= 0) {
                                B = hmul8(B, hfrag(HD, cf, kb));
                            }
                            mma16(acc[t], A, B);
                        }
                        if (t < 16 / NKB) issue_tok(cn, kb * (16 / NKB) + t);
                    }
#pragma unroll
                    for (int u = NT; u < 16 / NKB; ++u) issue_tok(cn, kb * (16 / NKB) + u);
                }
                // the wave's two diagonal blocks 2h, 2h + 1 (one inlined copy of the exact path)
#pragma nounroll
                for (int d = 0; d < 2; ++d) {
                    const int b = 2 * h + d;
                    if (fl[b]) {
                        const float4v x = diag_exact(isQ ? rq : rk, c, b, GD2 && !isQ);
#pragma unroll
                        for (int t = 0; t < NT; ++t)
                            if (cf_[h][t] == 3) acc[t] = ti_[h][t] == b ? x : acc[t];
                    }
                }
            }
            // epilogue: beta of the row for N (not for GD2: e carries the gate), causal masks
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int ti = ti_[h][t], tj = tj_[h][t];
                const int m = 16 * tj + j, l0 = 16 * ti + 4 * g;
                float v[4];
                if (!isQ && !GD2) {
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
        };
        // The test for the exact diagonal path is taken once per wave, so the usual all-fp16
        // case runs as straight-line code (a branch inside the loop serialises its LDS reads).
        auto gram_wave = [&](auto hc, auto qc) {
            constexpr int h = decltype(hc)::value;
            if (__builtin_amdgcn_readfirstlane(Flag[2 * h] | Flag[2 * h + 1]))
                gram_kda(hc, qc, std::true_type{});
            else
                gram_kda(hc, qc, std::false_type{});
        };
        if (w == 0) gram_wave(std::integral_constant<int, 0>{}, std::false_type{});
        else if (w == 1) gram_wave(std::integral_constant<int, 1>{}, std::false_type{});
        else if (w == 2) gram_wave(std::integral_constant<int, 0>{}, std::true_type{});
        else gram_wave(std::integral_constant<int, 1>{}, std::true_type{});
        lds_barrier();

        // Diagonal inverses (waves 0-1, two blocks each): column-oriented forward substitution,
        // lane (block, jc) builds column jc of X_bb = N_bb^{-1}, stored as X_bb^T (row jc =
        // column jc), and the diagonal block of T = N^{-1} diag(beta) (GD2: N^{-1}, e carries
        // the gate) into Tt.
        auto diag_inverse = [&]() {
            const int b = 2 * w + ((l >> 4) & 1), jc = j;
            const float* nb = Nd + b * 16 * L::LDN;
            float4v nr[15][4];
#pragma unroll
            for (int i = 0; i < 15; ++i)
#pragma unroll
                for (int q4 = (i + 1) / 4; q4 < 4; ++q4) nr[i][q4] = ld4f(nb + i * L::LDN + 4 * q4);
            float xd[16];
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
            if (l < 32) {
                half8 h0, h1;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    h0[t] = (_Float16)xd[t];
                    h1[t] = (_Float16)xd[8 + t];
                }
                *reinterpret_cast<half8*>(Xd + (16 * b + jc) * L::LDX) = h0;
                *reinterpret_cast<half8*>(Xd + (16 * b + jc) * L::LDX + 8) = h1;
                const float bc = GD2 ? 1.0f : FB[16 * b + jc];
                const int pc = pperm(16 * b + jc);
#pragma unroll
                for (int i = 0; i < 16; ++i) Tt[(16 * b + i) * L::LDC + pc] = (_Float16)(xd[i] * bc);
            }
        };

        // The chunk's operands go to the workspace in 16-byte pieces, spread over the last
        // stages: waves 2-3 write K e^G and Q e^G while waves 0-1 invert the diagonal blocks,
        // then K e^{G_C - G} while waves 0-1 form the blocks below the diagonal; all waves
        // then write A^T, T and e^{G_C}.  The copies are rescaled on the way out (per block
        // and channel: e^{G_start(blk)} for Kr and Qr, e^{G_C - G_end(blk)} for Kc).
        uint16_t* dst = a.ws + (bh * nC + c) * (int64_t)kda_ws_stride<DK>();
        constexpr int NG = C * (DK / 8);  // 16-byte pieces per copy
        auto copy_scaled = [&](const _Float16* src, const _Float16* H, uint16_t* d) {
#pragma unroll
            for (int u = 0; u < NG / 128; ++u) {
                const int i = tid - 128 + 128 * u;
                const int row = i / (DK / 8), col = (i % (DK / 8)) * 8;
                *reinterpret_cast<half8*>(d + row * DK + col) =
                    hmul8(ld8(src + row * L::LDK + col), ld8(H + (row >> 4) * DK + col));
            }
        };
        if (w < 2) {
            diag_inverse();
        } else {
            copy_scaled(Kr, HP, dst + 2 * kTriHalfs);
            copy_scaled(Qr, HP, dst + 2 * kTriHalfs + C * DK);
        }
        lds_barrier();
        // blocks of N^{-1} below the diagonal, column block by column block (wave 0: column
        // 0, wave 1: columns 1 and 2): M_bc = -X_bb sum_{d=c}^{b-1} N_bd M_dc, then
        // T_bc = M_bc diag(beta_c)
        auto mma16k16 = [](float4v& acc4, const half4& a4, const half4& b4) {
            acc4 = __builtin_amdgcn_mfma_f32_16x16x16f16(a4, b4, acc4, 0, 0, 0);
        };
        auto h4 = [](const float4v& x) { return half4{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]}; };
        auto xA = [&](int b) { return ldtr(Xd + (16 * b + 4 * g + (j >> 2)) * L::LDX + 4 * (j & 3)); };
        auto nA = [&](int b, int d) { return ldtr(Nt + (16 * d + 4 * g + (j >> 2)) * L::LDC + 16 * b + 4 * (j & 3)); };
        auto column = [&](auto cc) {
            constexpr int cb = decltype(cc)::value;
            half4 mb[4];
            mb[cb] = *reinterpret_cast<const half4*>(Xd + (16 * cb + j) * L::LDX + 4 * g);
            const float bcol = GD2 ? 1.0f : FB[16 * cb + j];
            const int pc = pperm(16 * cb + j);
#pragma unroll
            for (int b = cb + 1; b < 4; ++b) {
                float4v y = zero4();
#pragma unroll
                for (int d = cb; d < b; ++d) mma16k16(y, nA(b, d), mb[d]);
                float4v m = zero4();
                mma16k16(m, xA(b), h4(y));
#pragma unroll
                for (int r = 0; r < 4; ++r) m[r] = -m[r];
                mb[b] = h4(m);
#pragma unroll
                for (int r = 0; r < 4; ++r) Tt[(16 * b + 4 * g + r) * L::LDC + pc] = (_Float16)(m[r] * bcol);
            }
        };
        if (w == 0) {
            column(std::integral_constant<int, 0>{});
        } else if (w == 1) {
            column(std::integral_constant<int, 1>{});
            column(std::integral_constant<int, 2>{});
        } else {
            copy_scaled(Kc, HS, dst + 2 * kTriHalfs + 2 * C * DK);
        }
        lds_barrier();
        // A^T and T without their all-zero 32x32 blocks.  T's 16x16 blocks above the diagonal
        // are zero and are not staged: of a piece at column position col, the first four values
        // lie in 16-block column 2 (col / 32), the last four in the next one.
        for (int idx = tid; idx < kTriPieces; idx += 256) {
            int ra, ca, row, col;
            at_piece(idx, ra, ca);
            t_piece(idx, row, col);
            *reinterpret_cast<uint4*>(dst + idx * 8) = *reinterpret_cast<const uint4*>(At + ra * L::LDC + ca);
            uint4 t = *reinterpret_cast<const uint4*>(Tt + row * L::LDC + col);
            const int rb = row >> 4, cb = 2 * (col >> 5);
            if (cb > rb) t.x = t.y = 0u;
            if (cb + 1 > rb) t.z = t.w = 0u;
            *reinterpret_cast<uint4*>(dst + kTriHalfs + idx * 8) = t;
        }
        if (tid < DK) reinterpret_cast<float*>(dst + 2 * kTriHalfs + 3 * C * DK)[tid] = FE[tid];
        // No barrier before the next chunk: its scan and tables write nothing read here, and
        // Tt is written again only after three more barriers.
    }
}

template <int DK, bool GD2>
static hipError_t launch_kda(const KdaArgs& a, int64_t nwg, hipStream_t st) {
    using L = KdaLds<DK>;
    auto kern = chunk_kda_kernel<DK, GD2>;
    static std::atomic<uint64_t> lds_enabled{0};  // one bit per device
    if (const hipError_t e = enable_dynamic_lds(kern, L::total, lds_enabled); e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(256), L::total, st, a);
    return hipGetLastError();
}

// UT pass of the per-channel-gate two-kernel path: one group per (sequence, run of chunks), the
// runs sized so the grid about fills the chip once (a group walks its chunks with the next
// chunk's loads in flight).  With an erase gate eg (Gated DeltaNet-2) the row operand is
// eg (.) k and T = N^{-1}; beta is then unused.
hipError_t chunk_kda_ut_dispatch(int64_t BH, int64_t T, int dk, const void* q, const void* k, const float* g,
                                 const float* beta, const float* eg, void* ws, hipStream_t st) {
    KdaArgs a;
    a.T = T;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.g = g;
    a.beta = eg ? nullptr : beta;
    a.eg = eg;
    a.ws = static_cast<uint16_t*>(ws);
    const int64_t nC = (T + kChunk - 1) / kChunk;
    if (BH * nC == 0) return hipSuccess;
    int ncu = 1;
    if (const hipError_t e = device_cu_count(ncu); e != hipSuccess) return e;
    const int64_t cpw = (BH * nC + ncu - 1) / ncu;
    a.cpw = (int)(cpw < nC ? cpw : nC);
    const int64_t nwg = BH * ((nC + a.cpw - 1) / a.cpw);
    if (eg) {
        if (dk == 128) return launch_kda<128, true>(a, nwg, st);
        return launch_kda<64, true>(a, nwg, st);
    }
    if (dk == 128) return launch_kda<128, false>(a, nwg, st);
    return launch_kda<64, false>(a, nwg, st);
}

int64_t chunk_kda_ws_halfs(int dk) { return dk == 128 ? kda_ws_stride<128>() : kda_ws_stride<64>(); }

}  // namespace gdr
