// chunk_split.hip -- chunked forward of the gated delta rule (scalar gate, bf16 I/O) as two
// kernels: the chunk-local UT transform for every chunk at once, then the chunk-serial state
// pass.  gfx950, fp16 MFMA operands, fp32 accumulation and state.
//
// "Linear Attention, Visualized", section "Gated DeltaNet (GDN)", "Complete per-chunk
// algorithm" (column convention): within a chunk,
//   N = I + diag(beta) (K K^T (.) Gam)_strict,   T = N^{-1} diag(beta),   A = (Q K^T) (.) Gam
// depend on the chunk's own inputs only, and the page notes that they can be formed for all
// chunks in parallel before the boundary pass threads the state through the chunks.  So:
//
//   chunk_ut_kernel     one workgroup per (sequence, chunk), all chunks at once: the decay scan,
//                       the Gram tiles of K K^T and Q K^T, the four 16x16 diagonal blocks of
//                       N^{-1} by fp32 forward substitution, the blocks below the diagonal by
//                       16x16 MFMA products (M_bc = -X_bb sum_{c<=d<b} N_bd M_dc), and T and A
//                       written to a workspace as fp16 (12 KiB per chunk and sequence);
//   chunk_state_kernel  one workgroup per (sequence, 32 value channels), chunks in order:
//                       R = V - diag(e^G) K S^T,  Z = T R,  O = diag(e^G) Q S^T + A Z,
//                       S^T <- e^{G_C} S^T + K^T diag(e^{G_C - G}) Z.
//
// With T formed in advance, the serial chain of a chunk is three dependent product groups
// (K S^T, T R, the state update) instead of a blocked substitution, and the UT work is done
// once per chunk instead of once per value-channel tile.  The price is the workspace traffic
// (T and A written once and read by every value-channel tile) and a second read of K and Q.
//
// Workspace layout, per (sequence, chunk): A^T (row m holds A[l][m], l = 0..63), then T (row l;
// column m stored at position pperm(m), so one operand fragment is one 16-byte read), both fp16
// with zeros in the upper 16x16 blocks of their diagonal 32x32 blocks and their all-zero 32x32
// block left out (3072 halfs each, see at_piece / t_piece); then the decay factors of the state
// pass, fp32: e^{G_l} [64], e^{G_C - G_l} [64], e^{G_C}, 15 zeros (12864 bytes).  With the fused
// input preparation the state pass reads the raw q and k rows and takes their inverse norms in
// its per-token factors: e^{G_l}/||k_l||, e^{G_C - G_l}/||k_l||, e^{G_C}, 15 zeros and
// e^{G_l}/||q_l|| (13120 bytes); only the UT pass needs the normalised rows themselves.
//
// The per-channel gate ("Kimi Delta Attention (KDA)" section of the same page) takes the same
// state kernel in its KDA instantiation: the UT pass (chunk_kda.hip) also writes the decayed
// copies K e^G, Q e^G, K e^{G_C - G} and e^{G_C} per channel, so the state pass scales
// nothing itself:  R = V - (K e^G) S^T,  Z = T R,  O = (Q e^G) S^T + A Z,
// S^T <- Diag(e^{G_C}) S^T + (K e^{G_C - G})^T Z.  The loaders stage K e^G in the K buffer and
// K e^{G_C - G} in the Q buffer; the consumers read their Q e^G fragments straight from the
// workspace, one chunk ahead, and take the Q e^G S^T products after Z, off the serial chain.
// Gated DeltaNet-2 ("Gated DeltaNet-2, and the gate that was doing two jobs", section 2) runs
// the same code in its own instantiation: its UT pass has put the erase gate into the row copy
// (b (.) k) e^G and into T = N^{-1}, and the loaders stage z = w (.) v, computed and kept in
// fp32 (the V buffer's rows hold 32 fp32 channels), in place of V.
#include <type_traits>

#include "chunk_common.h"

namespace gdr {

// per-chunk factor table of the UT kernel (floats):
//   [0,64) G   [64,128) 1/||k_l||, [128,192) 1/||q_l|| (fused preparation)   [192,256) beta
//   [272,336) cf[m] = e^{Gend(blk(m)) - G_m}   [336,528) rf[b][l] = e^{G_l - Gend(b)}
//   [528,720) rb[b][l] = beta_l rf[b][l]
struct UtTab {
    static constexpr int SG = 0, SIK = 64, SIQ = 128, SB = 192, SCF = 272, SRF = 336, SRB = 528, NSM = 736;
};

// workspace record of one (sequence, chunk) of the scalar gate, in halfs: A^T, T, factors
constexpr int kGdnWsFactors = 2 * kTriHalfs;               // offset of the fp32 factor table
constexpr int kGdnWsNF = 144;                               // its floats
constexpr int kGdnWsStride = kGdnWsFactors + 2 * kGdnWsNF;  // 6432 halfs = 12864 bytes
// fused input preparation: the factor table holds e^G/||k|| [64], e^{G_C - G}/||k|| [64],
// e^{G_C}, 15 zeros, e^G/||q|| [64] (13120 bytes per record for either DK)
constexpr int kPrepNF = 208;
constexpr int kPrepWsStride = kGdnWsFactors + 2 * kPrepNF;

struct UtArgs {
    int H;              // PREP: heads (bh mod H is the head of the gate parameters)
    const float* A_log; // PREP: [H]
    const float* dt_bias;  // PREP: [H]
    int64_t T;          // steps per sequence (T_real n_h virtual steps for the VIRT kernels)
    int64_t Treal;      // rows of q and g per sequence (= T unless VIRT)
    uint32_t nh;        // substeps per token (VIRT)
    uint32_t nh_magic;  // ceil(2^32 / nh): m / nh = umulhi(m, nh_magic) for m < 2^23
    int64_t nC;
    const uint16_t* q;
    const uint16_t* k;
    const float* g;
    const float* beta;
    uint16_t* ws;
};

template <int DK>
struct UtLds {
    static constexpr int C = kChunk;
    static constexpr int LDK = DK + 16;  // halfs, rows of K / Q (conflict-free fragment reads)
    static constexpr int LDC = C + 8;    // halfs, rows of C-wide fp16 matrices
    static constexpr int LDN = 16 + 4;   // floats, rows of a 16x16 fp32 block
    static constexpr int LDX = 16 + 8;   // halfs, rows of a 16x16 fp16 block
    static constexpr int szK = C * LDK * 2;
    static constexpr int szC = C * LDC * 2;
    // K and Q during the Gram products; afterwards the same bytes hold N^T, A^T, T, the
    // diagonal blocks of N^T (fp32) and X_bb^T (fp16), all written after the last K and Q read
    static constexpr int oK = 0, oQ = szK;
    static constexpr int oNt = 0, oAt = szC, oTt = 2 * szC;
    static constexpr int oNd = 3 * szC;                       // diagonal blocks of N^T (fp32)
    static constexpr int oXd = oNd + 4 * 16 * LDN * 4;        // X_bb^T (fp16)
    static constexpr int endAfter = oXd + 4 * 16 * LDX * 2;
    static constexpr int szAlias = (2 * szK > endAfter ? 2 * szK : endAfter);
    static constexpr int oSm = (szAlias + 15) / 16 * 16;
    static constexpr int total = oSm + UtTab::NSM * 4;
    // four workgroups per CU at DK = 128 (39808 bytes each)
    static_assert(total <= 160 * 1024 / 4, "the UT kernel is sized for four workgroups per CU");
    static_assert((oSm | oNd | oXd | oAt | oTt) % 16 == 0, "alignment");
};

// Instantiations: plain, VIRT and PREP.
// VIRT: Gated Delta Product over its virtual steps ("Linear Attention, Visualized", "GDP as GDN
// over a virtual sequence"): step m = n_h t + j reads q_t only when j = n_h - 1 and g_t only
// when j = 0; other steps read past the end of the real-token buffer, which returns zero.
// PREP: the inputs from raw projections (same page, "Optional: Constructing the decay gate",
// and the unit-norm convention of keys and queries): q = q_raw / max(||q_raw||, 1e-6), k
// likewise, beta = sigmoid(beta_logit), g = -e^{A_log[h]} softplus(dt + dt_bias[h]); the
// inverse norms go into the state pass's per-token factors.
constexpr int kUtPlain = 0, kUtVirt = 1, kUtPrep = 2;
template <int DK, int UM>
__global__ __launch_bounds__(128) void chunk_ut_kernel(const UtArgs a) {
    constexpr bool VIRT = UM == kUtVirt, PREP = UM == kUtPrep;
    constexpr int WSS = PREP ? kPrepWsStride : kGdnWsStride;  // workspace halfs per chunk
    using L = UtLds<DK>;
    using S = UtTab;
    constexpr int C = kChunk;
    constexpr int NKB = DK / 32;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    _Float16* Kb = reinterpret_cast<_Float16*>(smem + L::oK);
    _Float16* Qb = reinterpret_cast<_Float16*>(smem + L::oQ);
    _Float16* Nt = reinterpret_cast<_Float16*>(smem + L::oNt);
    _Float16* At = reinterpret_cast<_Float16*>(smem + L::oAt);
    _Float16* Tt = reinterpret_cast<_Float16*>(smem + L::oTt);
    float* sm = reinterpret_cast<float*>(smem + L::oSm);
    float* Nd = reinterpret_cast<float*>(smem + L::oNd);
    _Float16* Xd = reinterpret_cast<_Float16*>(smem + L::oXd);

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, j = l & 15, g = l >> 4;
    const int64_t bh = blockIdx.x / a.nC;
    const int64_t c = blockIdx.x - bh * a.nC;
    const int64_t T = a.T;
    const int64_t Tr = VIRT ? a.Treal : T;
    const uint32_t t0 = (uint32_t)(c * C);
    const auto rq = make_rsrc(a.q + bh * Tr * DK, (uint32_t)(Tr * DK * 2));
    const auto rk = make_rsrc(a.k + bh * T * DK, (uint32_t)(T * DK * 2));
    const auto rg = make_rsrc(a.g + bh * Tr, (uint32_t)(Tr * 4));
    const auto rb = make_rsrc(a.beta + bh * T, (uint32_t)(T * 4));
    auto vtok = [&](uint32_t m) { return __umulhi(m, a.nh_magic); };

    // ---- K and Q of the chunk into LDS (fp16, natural channel order); past the sequence end
    // the loads return zeros, i.e. identity tokens
    constexpr int NP = C * DK / 8 / 128;  // 16-byte pieces per thread and matrix
    {
        uint4 kr[NP], qr[NP];
#pragma unroll
        for (int u = 0; u < NP; ++u) {
            const int idx = tid + 128 * u, row = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            const uint32_t off = ((t0 + row) * DK + col) * 2;
            uint32_t offq = off;
            if constexpr (VIRT) {
                const uint32_t m = t0 + row, tr = vtok(m);
                offq = m - tr * a.nh == a.nh - 1 ? (tr * DK + col) * 2 : (uint32_t)(Tr * DK * 2);
            }
            kr[u] = bld16(rk, off);
            qr[u] = bld16(rq, offq);
        }
        float gl = 0.0f, bt = 0.0f;
        if (w == 0) {
            uint32_t offg = (t0 + l) * 4;
            if constexpr (VIRT) {
                const uint32_t m = t0 + l, tr = vtok(m);
                offg = m - tr * a.nh == 0 ? tr * 4 : (uint32_t)(Tr * 4);
            }
            gl = bld4(rg, offg);
            bt = bld4(rb, (t0 + l) * 4);
            if constexpr (PREP) {  // past the sequence end: identity tokens (g = 0, beta = 0)
                const bool live = (int64_t)(t0 + l) < T;
                const int h = (int)(bh % a.H);
                const float lam = fast_exp(a.A_log[h]), z = gl + a.dt_bias[h];
                // softplus(z) = max(z, 0) + log(1 + e^{-|z|})
                gl = live ? -lam * (fmaxf(z, 0.0f) + __logf(1.0f + fast_exp(-fabsf(z)))) : 0.0f;
                bt = live ? 1.0f / (1.0f + fast_exp(-bt)) : 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < NP; ++u) {
            const int idx = tid + 128 * u, row = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            if constexpr (PREP) {
                // one row spans DK / 8 consecutive lanes: a DPP sum inside each 16-lane row
                float ik, iq;
                const half8 hk = unit_rows<DK>(kr[u], ik), hq = unit_rows<DK>(qr[u], iq);
                *reinterpret_cast<half8*>(Kb + row * L::LDK + col) = hk;
                *reinterpret_cast<half8*>(Qb + row * L::LDK + col) = hq;
                if (col == 0) {
                    sm[S::SIK + row] = ik;
                    sm[S::SIQ + row] = iq;
                }
            } else {
                *reinterpret_cast<half8*>(Kb + row * L::LDK + col) = bf16x8_to_half8(kr[u]);
                *reinterpret_cast<half8*>(Qb + row * L::LDK + col) = bf16x8_to_half8(qr[u]);
            }
        }
        // in-chunk cumulative log-decay and the factor table (wave 0, lane = token)
        if (w == 0) {
            const float x = wave_inclusive_scan(gl);
            float ge[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) ge[b] = lane_value(x, 16 * b + 15);
            const int blk = l >> 4;
            sm[S::SG + l] = x;
            // the state pass's factors of this chunk (PREP: after the barrier, with the norms)
            const float GC = ge[3];
            if constexpr (!PREP) {
                float* fw = reinterpret_cast<float*>(a.ws + (bh * a.nC + c) * WSS + kGdnWsFactors);
                fw[l] = fast_exp(x);
                fw[64 + l] = fast_exp(GC - x);
                if (l < kGdnWsNF - 128) fw[128 + l] = l == 0 ? fast_exp(GC) : 0.0f;
            }
            sm[S::SB + l] = bt;
            sm[S::SCF + l] = fast_exp(ge[blk] - x);
#pragma unroll
            for (int b = 0; b < 3; ++b) {
                const float f = blk > b ? fast_exp(x - ge[b]) : 0.0f;
                sm[S::SRF + 64 * b + l] = f;
                sm[S::SRB + 64 * b + l] = bt * f;
            }
        }
    }
    lds_barrier();
    if constexpr (PREP) {  // per-token factors with the inverse norms of the raw rows
        if (w == 0) {
            float* fw = reinterpret_cast<float*>(a.ws + (bh * a.nC + c) * WSS + kGdnWsFactors);
            const float x = sm[S::SG + l], GC = sm[S::SG + C - 1];
            const float ik = sm[S::SIK + l], eg = fast_exp(x);
            fw[l] = eg * ik;
            fw[64 + l] = fast_exp(GC - x) * ik;
            if (l < 16) fw[128 + l] = l == 0 ? fast_exp(GC) : 0.0f;
            fw[144 + l] = eg * sm[S::SIQ + l];
        }
    }

    // ---- Gram tiles.  Wave 0 forms KK {00,10,11,20,21,30,31} and QK {00,10,11}; wave 1 forms
    // KK {22,32,33} and QK {20,21,22,30,31,32,33}.  Off the diagonal the decay is factorised
    // through the 16-token block ends (both factors <= 1); on it it is exact.
    // The tile lists are indexed by the wave's role, so the role is a compile-time constant.
    auto gram = [&](auto pc) {
    constexpr int P = decltype(pc)::value;
    constexpr int NT = 10;
    constexpr int tq[2][NT] = {{0, 0, 0, 0, 0, 0, 0, 1, 1, 1}, {0, 0, 0, 1, 1, 1, 1, 1, 1, 1}};
    constexpr int ti_[2][NT] = {{0, 1, 1, 2, 2, 3, 3, 0, 1, 1}, {2, 3, 3, 2, 2, 2, 3, 3, 3, 3}};
    constexpr int tj_[2][NT] = {{0, 0, 1, 0, 1, 0, 1, 0, 0, 1}, {2, 2, 3, 0, 1, 2, 0, 1, 2, 3}};
    float4v acc[NT];
    float4v fr[NT];
    float fc[NT];
    {
        auto load6 = [&](half8* f, int kb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) f[r] = ld8(Kb + (16 * r + j) * L::LDK + 32 * kb + 8 * g);
#pragma unroll
            for (int r = 0; r < 2; ++r) f[4 + r] = ld8(Qb + (16 * (2 * P + r) + j) * L::LDK + 32 * kb + 8 * g);
        };
        auto factors = [&](const int t) {
            const int ti = ti_[P][t], tj = tj_[P][t];
            const bool isQ = tq[P][t];
            const int m = 16 * tj + j, l0 = 16 * ti + 4 * g;
            if (ti != tj) {
                fr[t] = ld4f(sm + (isQ ? S::SRF : S::SRB) + 64 * tj + l0);
                fc[t] = sm[S::SCF + m];
            } else {
                const float Gm = sm[S::SG + m];
                const float4v Gl = ld4f(sm + S::SG + l0);
                const float4v bl = isQ ? float4v{1.0f, 1.0f, 1.0f, 1.0f} : ld4f(sm + S::SB + l0);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool keep = isQ ? (m <= l0 + r) : (m < l0 + r);
                    fr[t][r] = keep ? bl[r] * fast_exp(Gl[r] - Gm) : 0.0f;
                }
                fc[t] = 1.0f;
            }
        };
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = zero4();
        half8 fa[6], fb[6];
        load6(fa, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            half8* cur = (kb & 1) ? fb : fa;
            half8* nxt = (kb & 1) ? fa : fb;
            if (kb + 1 < NKB) load6(nxt, kb + 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int ti = ti_[P][t], tj = tj_[P][t];
                const half8 A = tq[P][t] ? cur[4 + (ti - 2 * P)] : cur[ti];
                mma16(acc[t], A, cur[tj]);
            }
            if (kb < 2) {
#pragma unroll
                for (int t = 5 * kb; t < 5 * kb + 5; ++t) factors(t);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    lds_barrier();  // every read of K and Q is done: their bytes become N^T, A^T and T
    // Zeros where the record holds them and no later write lands: the 16x16 blocks of A^T
    // below the block diagonal inside the stored region (rows 16-31 x columns 0-15, rows 48-63
    // x columns 32-47), and the upper blocks of T's stored diagonal 32x32 blocks (rows 0-15
    // and 32-47 of their 32 stored columns; the inverses overwrite the diagonal 16x16 blocks
    // inside those rows later).  Every other element of A^T and T that the copy-out reads is
    // written by this epilogue, the inverses or the blocks below the diagonal; N^T is read
    // below its block diagonal only.  None of these stores meets another write before the
    // next barrier.
    for (int i = tid; i < 192; i += 128) {
        _Float16* z;
        if (i < 64) {
            const int r = i < 32 ? 16 + (i >> 1) : 48 + ((i - 32) >> 1), cz = (i < 32 ? 0 : 32) + (i & 1) * 8;
            z = At + r * L::LDC + cz;
        } else {
            const int k = i - 64, hi = k >> 6, kk = k & 63;
            z = Tt + (32 * hi + (kk >> 2)) * L::LDC + 32 * hi + (kk & 3) * 8;
        }
        *reinterpret_cast<uint4*>(z) = uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int ti = ti_[P][t], tj = tj_[P][t];
        const bool isQ = tq[P][t];
        const int m = 16 * tj + j, l0 = 16 * ti + 4 * g;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc[t][r] * fr[t][r] * fc[t];
        if (ti == tj && !isQ) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (m == l0 + r) v[r] = 1.0f;
            *reinterpret_cast<float4v*>(Nd + (ti * 16 + j) * L::LDN + 4 * g) = float4v{v[0], v[1], v[2], v[3]};
        } else {
            _Float16* dst = (isQ ? At : Nt) + m * L::LDC + l0;
            *reinterpret_cast<half4*>(dst) = half4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
        }
    }
    };
    if (w == 0) gram(std::integral_constant<int, 0>{});
    else gram(std::integral_constant<int, 1>{});
    lds_barrier();

    // ---- diagonal blocks X_bb = N_bb^{-1}: wave w takes blocks 2w, 2w+1, lane (block, jc)
    // builds column jc by forward substitution in fp32.  Stored as X_bb^T (fp16) for the
    // products below, and as the diagonal blocks of T = N^{-1} diag(beta).
    {
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
            const float bc = sm[S::SB + 16 * b + jc];
            const int pc = pperm(16 * b + jc);
#pragma unroll
            for (int i = 0; i < 16; ++i) Tt[(16 * b + i) * L::LDC + pc] = (_Float16)(xd[i] * bc);
        }
    }
    lds_barrier();

    // ---- blocks below the diagonal, column block by column block:
    //   M_bc = -X_bb sum_{d = c}^{b-1} N_bd M_dc   (M_cc = X_cc),   T_bc = M_bc diag(beta_c).
    // Wave 0 takes column 0 (three blocks), wave 1 columns 1 and 2.
    {
        auto mma16k16 = [](float4v& acc4, const half4& a4, const half4& b4) {
            acc4 = __builtin_amdgcn_mfma_f32_16x16x16f16(a4, b4, acc4, 0, 0, 0);
        };
        auto h4 = [](const float4v& x) { return half4{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]}; };
        // A operands (rows = lane j): X_bb from its transposed copy, N_bd from N^T
        auto xA = [&](int b) { return ldtr(Xd + (16 * b + 4 * g + (j >> 2)) * L::LDX + 4 * (j & 3)); };
        auto nA = [&](int b, int d) { return ldtr(Nt + (16 * d + 4 * g + (j >> 2)) * L::LDC + 16 * b + 4 * (j & 3)); };
        auto column = [&](auto cc) {
            constexpr int cb = decltype(cc)::value;
            half4 mb[4];
            mb[cb] = *reinterpret_cast<const half4*>(Xd + (16 * cb + j) * L::LDX + 4 * g);  // B operand X_cc
            const float bcol = sm[S::SB + 16 * cb + j];
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
        } else {
            column(std::integral_constant<int, 1>{});
            column(std::integral_constant<int, 2>{});
        }
    }
    lds_barrier();

    // ---- A^T and T to the workspace, 16-byte pieces, without their all-zero 32x32 blocks
    uint16_t* dst = a.ws + (bh * a.nC + c) * WSS;
#pragma unroll
    for (int u = 0; u < kTriPieces / 128; ++u) {
        const int idx = tid + 128 * u;
        int ra, ca, rt, ct;
        at_piece(idx, ra, ca);
        t_piece(idx, rt, ct);
        *reinterpret_cast<uint4*>(dst + idx * 8) = *reinterpret_cast<const uint4*>(At + ra * L::LDC + ca);
        *reinterpret_cast<uint4*>(dst + kTriHalfs + idx * 8) = *reinterpret_cast<const uint4*>(Tt + rt * L::LDC + ct);
    }
}

// ============================================================================ state pass

struct StArgs {
    int64_t T;          // steps per sequence (virtual steps for the GDP mode)
    int64_t Treal;      // rows of q and o per sequence (= T unless GDP)
    uint32_t nh;        // GDP: substeps per token
    uint32_t nh_magic;  // GDP: ceil(2^32 / nh)
    int64_t nC;
    int dv;
    int ntiles;  // d_v / (16 NCW)
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* wg;  // KDA mode: write gate w [T][dv] (Gated DeltaNet-2; V becomes w (.) v), or null
    const uint16_t* ws;
    const float* S0;
    uint16_t* o;
    float* Sf;
};

template <int DK>
struct StLds {
    static constexpr int C = kChunk;
    static constexpr int LDK = DK + 16;
    static constexpr int LDC = C + 8;
    static constexpr int LDV = 80;     // bf16, rows (tokens) of the 32-channel V tile
    static constexpr int LDO = C + 8;  // bf16, rows of O^T
    // factor table (scalar gate): [0,64) e^G   [64,128) e^{G_C - G}   [128] e^{G_C}
    // (per-channel gate: e^{G_C} [DK])
    static constexpr int FEG = 0, FER = 64, FEC = 128, FEQ = 144, NF = kGdnWsNF;
    // one 16-byte slot per loader thread, so that every loader lane stores its piece (the
    // slots past the table receive zeros) and no branch sits in the loaders' staging
    static constexpr int NFL = 128 * 4;
    static constexpr int szK = C * LDK * 2;
    static constexpr int szC = C * LDC * 2;
    static constexpr int szV = C * LDV * 2;
    static constexpr int oK = 0;                    // two buffers each
    static constexpr int oQ = oK + 2 * szK;
    static constexpr int oA = oQ + 2 * szK;
    static constexpr int oT = oA + 2 * szC;
    static constexpr int oV = oT + 2 * szC;
    static constexpr int oF = oV + 2 * szV;
    static constexpr int oOt = oF + 2 * NFL * 4;  // O^T of a chunk, two buffers
    static constexpr int szO = 32 * LDO * 2;
    static constexpr int total = oOt + 2 * szO;
    static_assert(total <= 160 * 1024, "LDS budget of one gfx950 CU exceeded");
    static_assert((oQ | oA | oT | oV | oF | oOt) % 16 == 0, "alignment");
};

// Modes of the state pass: the scalar gate, the per-channel gate (KDA), Gated DeltaNet-2
// (the KDA pass with z = w (.) v in place of v), and the Gated Delta Product (the scalar-gate
// pass over virtual steps: q read and o written on the last substep of a token only), and the
// fused input preparation (the scalar-gate pass over raw q and k, each row scaled by the
// inverse norm the UT pass wrote).
constexpr int kStGdn = 0, kStKda = 1, kStGd2 = 2, kStGdp = 3, kStPrep = 4;

// NCW consumer waves of 16 value channels each (a value tile of 16 NCW channels) and two loader
// waves.  NCW = 1 doubles the workgroups of a grid that would leave compute units idle.
template <int DK, int MODE, int NCW>
__global__ __launch_bounds__(64 * (NCW + 2), 1) void chunk_state_kernel(const StArgs a) {
    constexpr bool KDA = MODE == kStKda || MODE == kStGd2;  // the UT pass wrote the decayed copies
    constexpr bool ZW = MODE == kStGd2;                     // V tile holds z = w (.) v in fp32
    constexpr bool VIRT = MODE == kStGdp;                   // GDP virtual steps
    constexpr bool PREP = MODE == kStPrep;                  // raw q, k; inverse norms in the factors
    using L = StLds<DK>;
    constexpr int C = kChunk;
    constexpr int NKB = DK / 32;
    constexpr int NST = DK / 16;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    auto Kb = [&](int b) { return reinterpret_cast<_Float16*>(smem + L::oK + b * L::szK); };
    auto Qb = [&](int b) { return reinterpret_cast<_Float16*>(smem + L::oQ + b * L::szK); };
    auto Ab = [&](int b) { return reinterpret_cast<_Float16*>(smem + L::oA + b * L::szC); };
    auto Tb = [&](int b) { return reinterpret_cast<_Float16*>(smem + L::oT + b * L::szC); };
    auto Vb = [&](int b) { return reinterpret_cast<uint16_t*>(smem + L::oV + b * L::szV); };
    auto Fb = [&](int b) { return reinterpret_cast<float*>(smem + L::oF + b * L::NFL * 4); };
    auto Ob = [&](int b) { return reinterpret_cast<_Float16*>(smem + L::oOt + b * L::szO); };  // bf16 bits

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, j = l & 15, g = l >> 4;
    const bool consumer = w < NCW;
    // the consumers' chain is the critical path: let them win issue and LDS arbitration
    if (consumer) __builtin_amdgcn_s_setprio(2);
    const int vi = xcd_major_index(blockIdx.x, gridDim.x);
    const int64_t bh = vi / a.ntiles;
    const int dv0 = (vi % a.ntiles) * (16 * NCW);
    const int dvc = dv0 + 16 * w;
    const int64_t T = a.T, nC = a.nC;
    const int DV = a.dv;
    // (the per-channel gate reads no q or k: those resources are empty)
    const int64_t Tr = VIRT ? a.Treal : T;  // rows of q and o
    const auto rq = make_rsrc(KDA ? nullptr : a.q + bh * Tr * DK, KDA ? 0u : (uint32_t)(Tr * DK * 2));
    const auto rk = make_rsrc(KDA ? nullptr : a.k + bh * T * DK, KDA ? 0u : (uint32_t)(T * DK * 2));
    const auto rv = make_rsrc(a.v + bh * T * DV, (uint32_t)(T * DV * 2));
    const auto rwg = make_rsrc(ZW ? a.wg + bh * T * DV : nullptr, ZW ? (uint32_t)(T * DV * 4) : 0u);
    constexpr int WS = KDA ? kda_ws_stride<DK>() : PREP ? kPrepWsStride : kGdnWsStride;  // halfs per chunk
    // offsets (halfs) inside a chunk's workspace record of the per-channel gate
    constexpr int WKG = 2 * kTriHalfs, WQG = WKG + C * DK, WKC = WQG + C * DK, WFE = WKC + C * DK;
    const auto rw = make_rsrc(a.ws + bh * nC * WS, (uint32_t)(nC * WS * 2));
    const auto ro = make_rsrc(a.o + bh * Tr * DV, (uint32_t)(Tr * DV * 2));
    auto vtok = [&](uint32_t m) { return __umulhi(m, a.nh_magic); };

    auto trfrag = [&](const _Float16* base, int ld, int kb, int col) {
        const _Float16* p0 = base + (32 * kb + 4 * g + (j >> 2)) * ld + col;
        return cat8(ldtr(p0), ldtr(p0 + 16 * ld));
    };

    // ---- loader waves (the last two): two register sets, so a chunk's loads are issued two
    // chunks before the loaders stage it into LDS (one chunk ahead of the consumers)
    const int lt = tid - 64 * NCW;  // loader thread in [0, 128)
    constexpr int NPV = NCW;        // 16-byte pieces of the V tile per loader thread
    constexpr int NPK = C * DK / 8 / 128;  // K (and Q) pieces per loader thread
    constexpr int NPW = kTriPieces / 128;  // A^T (and T) pieces per loader thread
    // (KDA: kr holds K e^G, qr K e^{G_C - G}); fr: 16-byte pieces of the factor table, the
    // first NFQ loader threads one each
    constexpr int NFQ = KDA ? DK / 4 : PREP ? kPrepNF / 4 : L::NF / 4;
    struct LdRegs {
        uint4 kr[NPK], qr[NPK], ar[NPW], tr[NPW], vr[NPV], fr;
        uint4 wr[ZW ? 2 * NPV : 1];  // the write gate of the V pieces (Gated DeltaNet-2)
    };
    LdRegs R0, R1;
    // The loads of one chunk in two parts: part 0 (K, A^T, V) right after the set is staged,
    // part 1 (Q, T, the factor table) at the start of the next step, after the o stores, so that
    // the stores do not queue behind the whole chunk's loads in the CU's memory pipeline.
    auto issue_part = [&](auto pc, LdRegs& R, int64_t c) {
        constexpr int P = decltype(pc)::value;
        uint4 *kr = R.kr, *qr = R.qr, *ar = R.ar, *tr = R.tr, *vr = R.vr;
        const uint32_t t0 = (uint32_t)(c * C);
        const uint32_t wb = (uint32_t)(c * WS);
#pragma unroll
        for (int u = 0; u < NPK; ++u) {
            const int idx = lt + 128 * u, row = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            if constexpr (KDA) {
                if constexpr (P == 0) kr[u] = bld16(rw, (wb + WKG + idx * 8) * 2);
                else qr[u] = bld16(rw, (wb + WKC + idx * 8) * 2);
            } else {
                const uint32_t off = ((t0 + row) * DK + col) * 2;
                if constexpr (P == 0) {
                    kr[u] = bld16(rk, off);
                } else {
                    uint32_t offq = off;
                    if constexpr (VIRT) {  // q_t on the last substep of token t, zero elsewhere
                        const uint32_t m = t0 + row, tr = vtok(m);
                        offq = m - tr * a.nh == a.nh - 1 ? (tr * DK + col) * 2 : (uint32_t)(Tr * DK * 2);
                    }
                    qr[u] = bld16(rq, offq);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < NPW; ++u) {
            const int idx = lt + 128 * u;
            if constexpr (P == 0) ar[u] = bld16(rw, (wb + idx * 8) * 2);
            else tr[u] = bld16(rw, (wb + kTriHalfs + idx * 8) * 2);
        }
        if constexpr (P == 0) {
#pragma unroll
            for (int u = 0; u < NPV; ++u) {
                const int idx = lt + 128 * u, row = idx / (2 * NCW), col = (idx % (2 * NCW)) * 8;
                vr[u] = bld16(rv, ((t0 + row) * DV + dv0 + col) * 2);
                if constexpr (ZW) {
                    R.wr[2 * u] = bld16(rwg, ((t0 + row) * DV + dv0 + col) * 4);
                    R.wr[2 * u + 1] = bld16(rwg, ((t0 + row) * DV + dv0 + col) * 4 + 16);
                }
            }
        } else {
            // every loader lane loads (lanes past the table read past the buffer end: zeros), so
            // that no branch hides a load from the compiler's count of loads in flight
            R.fr = bld16(rw, lt < NFQ ? (wb + (KDA ? WFE : kGdnWsFactors)) * 2 + lt * 16 : (uint32_t)(nC * WS * 2));
        }
    };
    auto issue = [&](LdRegs& R, int64_t c) {
        issue_part(std::integral_constant<int, 0>{}, R, c);
        issue_part(std::integral_constant<int, 1>{}, R, c);
    };
    // o of chunk c from its O^T buffer: loader wave lw takes rows (value channels) 16 lw ..,
    // a lane reads 8 consecutive channels of one token back transposed and stores 16 bytes
    auto store_o = [&](int64_t c) {
        const int lw = w - NCW;
        if (NCW == 1 && lw >= NCW) return;  // 16-channel tiles: the second loader wave has no rows
        const _Float16* Ot = Ob((int)(c & 1));
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int tb = 32 * s2 + 16 * (g >> 1), d = 16 * lw + 8 * (g & 1);
            const _Float16* rp = Ot + (d + (j >> 2)) * L::LDO + tb + 4 * (j & 3);
            const uint2 lo = __builtin_bit_cast(uint2, ldtr(rp));
            const uint2 hi = __builtin_bit_cast(uint2, ldtr(rp + 4 * L::LDO));
            uint32_t offo = ((uint32_t)(c * C + tb + j) * DV + dv0 + d) * 2;
            if constexpr (VIRT) {  // only the last substep of a token has an output
                const uint32_t m = (uint32_t)(c * C + tb + j), tr = vtok(m);
                offo = m - tr * a.nh == a.nh - 1 ? (tr * DV + dv0 + d) * 2 : (uint32_t)(Tr * DV * 2);
            }
            bst16(ro, offo, uint4{lo.x, lo.y, hi.x, hi.y});
        }
    };
    // K and Q to fp16 in the registers (while the consumers' first products read LDS)
    auto convert = [&](LdRegs& R) {
        if constexpr (KDA) return;  // the UT pass wrote fp16
        uint4 *kr = R.kr, *qr = R.qr;
#pragma unroll
        for (int u = 0; u < NPK; ++u) {
            kr[u] = __builtin_bit_cast(uint4, bf16x8_to_half8(kr[u]));
            qr[u] = __builtin_bit_cast(uint4, bf16x8_to_half8(qr[u]));
        }
    };
    auto stage = [&](LdRegs& R, int64_t c) {
        const uint4 *kr = R.kr, *qr = R.qr, *ar = R.ar, *tr = R.tr, *vr = R.vr;
        const int b = (int)(c & 1);
#pragma unroll
        for (int u = 0; u < NPK; ++u) {
            const int idx = lt + 128 * u, row = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            *reinterpret_cast<uint4*>(Kb(b) + row * L::LDK + col) = kr[u];
            *reinterpret_cast<uint4*>(Qb(b) + row * L::LDK + col) = qr[u];
        }
#pragma unroll
        for (int u = 0; u < NPW; ++u) {  // the all-zero 32x32 blocks are never read: not staged
            const int idx = lt + 128 * u;
            int ra, ca, rt, ct;
            at_piece(idx, ra, ca);
            t_piece(idx, rt, ct);
            *reinterpret_cast<uint4*>(Ab(b) + ra * L::LDC + ca) = ar[u];
            *reinterpret_cast<uint4*>(Tb(b) + rt * L::LDC + ct) = tr[u];
        }
#pragma unroll
        for (int u = 0; u < NPV; ++u) {
            const int idx = lt + 128 * u, row = idx / (2 * NCW), col = (idx % (2 * NCW)) * 8;
            if constexpr (ZW) {  // z = w (.) v in fp32: row `row` of the fp32 tile, 8 channels
                const uint32_t x[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
                const uint32_t wv[8] = {R.wr[2 * u].x, R.wr[2 * u].y, R.wr[2 * u].z, R.wr[2 * u].w,
                                        R.wr[2 * u + 1].x, R.wr[2 * u + 1].y, R.wr[2 * u + 1].z, R.wr[2 * u + 1].w};
                float z[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    z[2 * e] = __uint_as_float(x[e] << 16) * __uint_as_float(wv[2 * e]);
                    z[2 * e + 1] = __uint_as_float(x[e] & 0xffff0000u) * __uint_as_float(wv[2 * e + 1]);
                }
                float* vf = reinterpret_cast<float*>(Vb(b)) + row * (L::LDV / 2) + col;
                *reinterpret_cast<float4v*>(vf) = float4v{z[0], z[1], z[2], z[3]};
                *reinterpret_cast<float4v*>(vf + 4) = float4v{z[4], z[5], z[6], z[7]};
            } else {
                *reinterpret_cast<uint4*>(Vb(b) + row * L::LDV + col) = vr[u];
            }
        }
        reinterpret_cast<uint4*>(Fb(b))[lt] = R.fr;
    };

    // ---- consumer waves (0, 1): the state S^T of 16 value channels (fp32 accumulators, rows
    // permuted by pperm) and its fp16 operand copy
    float4v St[NST];
    half8 Sb[NKB];
#pragma unroll
    for (int t = 0; t < NST; ++t) St[t] = zero4();
    if (consumer && a.S0 != nullptr) {
        const float* s0 = a.S0 + bh * (int64_t)DV * DK + (int64_t)(dvc + j) * DK;
#pragma unroll
        for (int t = 0; t < NST; ++t) St[t] = ld4f(s0 + pperm(16 * t + 4 * g));
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) Sb[kb] = pack8(St[2 * kb], St[2 * kb + 1]);
    // Operand range: the consumers hold S, R and Z multiplied by 2^sexp (one exponent per wave,
    // the same for all of its value channels).  Every step is linear in (V, S), so the scaled
    // quantities obey the same recurrence exactly; only the fp16 roundings see the scale, which
    // keeps max(|S|, |V|) 2^sexp inside [2^-3, 2^6] (rescaled to [2^3, 2^4) when it leaves it):
    // fp16's 11-bit mantissa then holds the values that matter, and no operand (|R| and |Z| stay
    // within a small multiple of that bound) reaches the fp16 maximum.  o and the final state
    // are divided by 2^sexp on the way out.  The test is lane-local plus a ballot; only a
    // rescale (rare) reduces across the wave.
    int sexp = 0;
    float ls = max_abs(St);  // this lane's largest |S| 2^sexp

    // Chunk k's loads live in register set k mod 2.  Loads of chunks past the end are issued
    // anyway (they read past the buffers' ends, which returns zeros, and are staged into a
    // buffer no consumer reads): with no branch around them the compiler can count the loads
    // in flight exactly, and waits for one set while the other stays in flight.
    if (!consumer && nC > 0) {
        issue(R0, 0);
        convert(R0);
        stage(R0, 0);
        issue(R1, 1);
        issue(R0, 2);
    }
    lds_barrier();

    // The two roles run separate loops with the same barrier sequence, so that the loaders'
    // prefetch registers are not live in the consumers' code (and the other way round).
    if (consumer) {
    // KDA: the chunk's Q e^G fragments (row 16 ti + j, channels 32 kb + 8 g ..), from the
    // workspace one chunk ahead
    half8 qg[KDA ? 4 : 1][KDA ? NKB : 1];
    auto issue_qg = [&](int64_t c) {
        if constexpr (KDA) {
            const uint32_t base = (uint32_t)(c * WS) + WQG;
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
                    qg[ti][kb] = __builtin_bit_cast(half8, bld16(rw, (base + (16 * ti + j) * DK + 32 * kb + 8 * g) * 2));
        }
    };
    if (nC > 0) issue_qg(0);
    // Per-channel modes: warm L2 ahead of the loaders.  The 8 consumer waves of a sequence (its
    // value tiles) each touch one 8 KiB slice of chunk c+3 (the 66 KB workspace record and the
    // V rows), one dword per 128-byte line; the result is folded into a sink a chunk later,
    // when the load has long returned.
    const int treg = ((vi % a.ntiles) * NCW + w) & 7;
    uint32_t tsink = 0, tch = 0;
    auto touch = [&](int64_t cc) {
        if constexpr (KDA) {
            const uint32_t line = (uint32_t)l * 128u;
            if (treg < 6)
                tch = __builtin_amdgcn_raw_buffer_load_b32(rw, (uint32_t)(cc * WS) * 2 + (uint32_t)treg * 8192u + line, 0, 0);
            else
                tch = __builtin_amdgcn_raw_buffer_load_b32(rv, (uint32_t)(cc * C) * DV * 2 + (uint32_t)(treg & 1) * 8192u + line, 0, 0);
        }
    };
    for (int64_t c = 0; c < nC; ++c) {
        const int bc = (int)(c & 1);
        if constexpr (KDA) {
            tsink ^= tch;
            touch(c + 3);
        }
        {
            const _Float16* Kc = Kb(bc);
            const _Float16* Qc = Qb(bc);
            const _Float16* Ac = Ab(bc);
            const _Float16* Tc = Tb(bc);
            const uint16_t* Vc = Vb(bc);
            const float* F = Fb(bc);
            auto kfrag = [&](int ti, int kb) { return ld8(Kc + (16 * ti + j) * L::LDK + 32 * kb + 8 * g); };
            auto qfrag = [&](int ti, int kb) { return ld8(Qc + (16 * ti + j) * L::LDK + 32 * kb + 8 * g); };
            // P_K = K S^T (rows = tokens), the head of the serial chain
            float4v PK[4];
            half8 fa[4], fb[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                PK[ti] = zero4();
                fa[ti] = kfrag(ti, 0);
            }
            // fragments that do not depend on the state (T, A, K^T) are loaded while the
            // first products run
            half8 tf[6], af[6];
            // K^T fragments (KDA: of K e^{G_C - G}, staged in the Q buffer)
            auto ktfrag = [&](int t, int kb) { return trfrag(KDA ? Qc : Kc, L::LDK, kb, pperm(16 * t + 4 * (j & 3))); };
            half8 kt0[NST], kt1[NST];
            auto prefetch = [&](int kb) {
                if (kb == 0) {
#pragma unroll
                    for (int ti = 0, n = 0; ti < 4; ++ti) {
#pragma unroll
                        for (int k2 = 0; k2 <= (ti >> 1); ++k2, ++n) {
                            tf[n] = ld8(Tc + (16 * ti + j) * L::LDC + 32 * k2 + 8 * g);
                            af[n] = trfrag(Ac, L::LDC, k2, 16 * ti + 4 * (j & 3));
                        }
                    }
                } else {
                    // K^T fragments: NST / (NKB - 1) tiles per later block
                    constexpr int PER = (NST + NKB - 2) / (NKB - 1);
#pragma unroll
                    for (int t = (kb - 1) * PER; t < kb * PER && t < NST; ++t) {
                        kt0[t] = ktfrag(t, 0);
                        kt1[t] = ktfrag(t, 1);
                    }
                }
            };
            float4v eg[4], vv[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                eg[ti] = KDA ? float4v{1.0f, 1.0f, 1.0f, 1.0f} : ld4f(F + L::FEG + 16 * ti + 4 * g);
                if constexpr (ZW) {  // fp32 tile [token][LDV / 2]
                    const float* vf = reinterpret_cast<const float*>(Vc) + (16 * ti + 4 * g) * (L::LDV / 2) + 16 * w + j;
#pragma unroll
                    for (int r = 0; r < 4; ++r) vv[ti][r] = vf[r * (L::LDV / 2)];
                } else {
                    const uint2 vb = __builtin_bit_cast(
                        uint2, ldtr(reinterpret_cast<const _Float16*>(Vc) + (16 * ti + 4 * g + (j >> 2)) * L::LDV +
                                    16 * w + 4 * (j & 3)));
                    vv[ti] = float4v{__uint_as_float(vb.x << 16), __uint_as_float(vb.x & 0xffff0000u),
                                     __uint_as_float(vb.y << 16), __uint_as_float(vb.y & 0xffff0000u)};
                }
            }
            const float lv = max_abs(vv);  // this lane's largest |V| of the chunk (unscaled)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                half8* cur = (kb & 1) ? fb : fa;
                half8* nxt = (kb & 1) ? fa : fb;
                if (kb + 1 < NKB) {
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti) nxt[ti] = kfrag(ti, kb + 1);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) mma16(PK[ti], cur[ti], Sb[kb]);
                prefetch(kb);
                __builtin_amdgcn_sched_barrier(0);
            }
            // the first block of Q fragments, for the products after Z
            half8 qa[4], qb[4];
            if constexpr (!KDA) {
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) qa[ti] = qfrag(ti, 0);
            }
            float4v er[4];
            float4v ed[KDA ? NST : 1];  // KDA: e^{G_C} of the state rows
            float eGC = 1.0f;
            if constexpr (KDA) {
#pragma unroll
                for (int t = 0; t < NST; ++t) ed[t] = ld4f(F + pperm(16 * t + 4 * g));
            } else {
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) er[ti] = ld4f(F + L::FER + 16 * ti + 4 * g);
                eGC = F[L::FEC];
            }
            __builtin_amdgcn_sched_barrier(0);
            // the operand scale of this chunk: when the chunk's V or the state leave the range
            // (a wave-uniform, rare branch), rescale S, repack its operand copy and redo P_K
            {
                const float lm = fmaxf(ls, lv * __builtin_ldexpf(1.0f, sexp));
                if (__any(lm > 64.0f) || __all(lm < 0.125f)) {
                    const float M = wave_max_abs(lm);
                    const int e2 = min(max(sexp + 4 - __builtin_amdgcn_frexp_expf(M), -100), 100);
                    if (M > 0.0f && M <= 3.0e38f && e2 != sexp) {
                        const float rho = __builtin_ldexpf(1.0f, e2 - sexp);
#pragma unroll
                        for (int t = 0; t < NST; ++t)
#pragma unroll
                            for (int r = 0; r < 4; ++r) St[t][r] *= rho;
#pragma unroll
                        for (int kb = 0; kb < NKB; ++kb) Sb[kb] = pack8(St[2 * kb], St[2 * kb + 1]);
#pragma unroll
                        for (int ti = 0; ti < 4; ++ti) PK[ti] = zero4();
#pragma unroll
                        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                            for (int ti = 0; ti < 4; ++ti) mma16(PK[ti], kfrag(ti, kb), Sb[kb]);
                        sexp = e2;
                    }
                }
            }
            const float vsc = __builtin_ldexpf(1.0f, sexp), osc = __builtin_ldexpf(1.0f, -sexp);
            // R = V - e^G P_K (scaled)
            float4v Rr[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int r = 0; r < 4; ++r) Rr[ti][r] = vv[ti][r] * vsc - eg[ti][r] * PK[ti][r];
            // Z = T R (T lower triangular: block column kb only for row tiles ti >= 2 kb)
            const half8 rB[2] = {pack8(Rr[0], Rr[1]), pack8(Rr[2], Rr[3])};
            float4v Zz[4];
#pragma unroll
            for (int ti = 0, n = 0; ti < 4; ++ti) {
                Zz[ti] = zero4();
#pragma unroll
                for (int kb = 0; kb <= (ti >> 1); ++kb, ++n) mma16(Zz[ti], tf[n], rB[kb]);
            }
            // S^T <- e^{G_C} S^T + K^T diag(e^{G_C - G}) Z first (the chain), then, off the
            // chain, P_Q = Q S^T with the state of the chunk start (its fp16 copy Sb) and
            // O = e^G P_Q + A Z
            const half8 zB[2] = {pack8(Zz[0], Zz[1]), pack8(Zz[2], Zz[3])};
            half8 sZ0 = zB[0], sZ1 = zB[1];
            if constexpr (!KDA) {
                float4v zs[4];
#pragma unroll
                for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                    for (int r = 0; r < 4; ++r) zs[ti][r] = er[ti][r] * Zz[ti][r];
                sZ0 = pack8(zs[0], zs[1]);
                sZ1 = pack8(zs[2], zs[3]);
            }
#pragma unroll
            for (int t = 0; t < NST; ++t) {
#pragma unroll
                for (int r = 0; r < 4; ++r) St[t][r] *= KDA ? ed[t][r] : eGC;
                mma16(St[t], kt0[t], sZ0);
                mma16(St[t], kt1[t], sZ1);
            }
            float4v PQ[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) PQ[ti] = zero4();
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                if constexpr (KDA) {
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti) mma16(PQ[ti], qg[ti][kb], Sb[kb]);
                } else {
                    half8* cur = (kb & 1) ? qb : qa;
                    half8* nxt = (kb & 1) ? qa : qb;
                    if (kb + 1 < NKB) {
#pragma unroll
                        for (int ti = 0; ti < 4; ++ti) nxt[ti] = qfrag(ti, kb + 1);
                    }
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti) mma16(PQ[ti], cur[ti], Sb[kb]);
                }
            }
            issue_qg(c + 1);  // past the end: zeros, unused (no branch: see the loaders)
            if constexpr (PREP) {  // the output's factor carries 1/||q|| instead of 1/||k||
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) eg[ti] = ld4f(F + L::FEQ + 16 * ti + 4 * g);
            }
            float4v Oa[4];
#pragma unroll
            for (int ti = 0, n = 0; ti < 4; ++ti) {
#pragma unroll
                for (int r = 0; r < 4; ++r) Oa[ti][r] = eg[ti][r] * PQ[ti][r];
#pragma unroll
                for (int kb = 0; kb <= (ti >> 1); ++kb, ++n) mma16(Oa[ti], af[n], zB[kb]);
            }
            // O unscaled and rounded to bf16 into this wave's rows of O^T (the loaders store it)
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
                *reinterpret_cast<uint2*>(Ob(bc) + (16 * w + j) * L::LDO + 16 * ti + 4 * g) =
                    uint2{pack_bf16x2(Oa[ti][0] * osc, Oa[ti][1] * osc), pack_bf16x2(Oa[ti][2] * osc, Oa[ti][3] * osc)};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) Sb[kb] = pack8(St[2 * kb], St[2 * kb + 1]);
            ls = max_abs(St);
        }
        lds_barrier();
    }
    if constexpr (KDA) {
        tsink ^= tch;
        asm volatile("" ::"v"(tsink));  // keeps the touches
    }
    } else {
    // loaders, step c (one per chunk, as the consumers' barriers): o of chunk c-1, part 1 of
    // chunk c+2 (into the other set), chunk c+1 (set (c+1) mod 2) into LDS, then part 0 of
    // chunk c+3 into the freed set
    auto step = [&](LdRegs& R, LdRegs& Ro, int64_t c) {
        store_o(c - 1);
        issue_part(std::integral_constant<int, 1>{}, Ro, c + 2);  // the rest of chunk c+2
        convert(R);
        stage(R, c + 1);
        issue_part(std::integral_constant<int, 0>{}, R, c + 3);
        lds_barrier();
    };
    if (nC > 0) {  // step 0 has no o to store (chunk 2 went out whole)
        convert(R1);
        stage(R1, 1);
        issue_part(std::integral_constant<int, 0>{}, R1, 3);
        lds_barrier();
    }
    int64_t c = 1;
    for (; c + 1 < nC; c += 2) {
        step(R0, R1, c);
        step(R1, R0, c + 1);
    }
    if (c < nC) step(R0, R1, c);
    if (nC > 0) store_o(nC - 1);
    }

    if (consumer && a.Sf != nullptr) {
        float* sf = a.Sf + bh * (int64_t)DV * DK + (int64_t)(dvc + j) * DK;
        const float osc = __builtin_ldexpf(1.0f, -sexp);
#pragma unroll
        for (int t = 0; t < NST; ++t) {
            float4v x = St[t];
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] *= osc;
            *reinterpret_cast<float4v*>(sf + pperm(16 * t + 4 * g)) = x;
        }
    }
}

template <int DK, int MODE, int NCW>
static hipError_t launch_state_ncw(StArgs s, int64_t BH, hipStream_t st) {
    using LS = StLds<DK>;
    auto ks = chunk_state_kernel<DK, MODE, NCW>;
    static std::atomic<uint64_t> lds_enabled{0};  // one bit per device
    if (const hipError_t e = enable_dynamic_lds(ks, LS::total, lds_enabled); e != hipSuccess) return e;
    s.ntiles = s.dv / (16 * NCW);
    hipLaunchKernelGGL(ks, dim3((unsigned)(BH * s.ntiles)), dim3(64 * (NCW + 2)), LS::total, st, s);
    return hipGetLastError();
}

// Value tiles of 32 channels, or of 16 when 32-channel tiles would leave compute units idle
// (one workgroup fills a compute unit's LDS).
template <int DK, int MODE>
static hipError_t launch_state(const StArgs& s, int64_t BH, hipStream_t st) {
    int ncu = 1;
    if (const hipError_t e = device_cu_count(ncu); e != hipSuccess) return e;
    if (BH * (s.dv / 32) < ncu) return launch_state_ncw<DK, MODE, 1>(s, BH, st);
    return launch_state_ncw<DK, MODE, 2>(s, BH, st);
}

template <int DK, int UM>
static hipError_t launch_split(const UtArgs& u, const StArgs& s, int64_t BH, hipStream_t st) {
    using LU = UtLds<DK>;
    auto ku = chunk_ut_kernel<DK, UM>;
    if (u.nC > 0) hipLaunchKernelGGL(ku, dim3((unsigned)(BH * u.nC)), dim3(128), LU::total, st, u);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_state<DK, UM == kUtVirt ? kStGdp : UM == kUtPrep ? kStPrep : kStGdn>(s, BH, st);
}

// Bytes of workspace the two-kernel path needs: 12864 per (sequence, chunk).
int64_t chunk_split_workspace_bytes(int64_t BH, int64_t T) {
    const int64_t nC = (T + kChunk - 1) / kChunk;
    return BH * nC * kGdnWsStride * 2;
}

// T counts real tokens; nh > 1 runs a Gated Delta Product over the T nh virtual steps (k, v,
// beta hold T nh rows per sequence; q, g, o hold T).  The workspace covers the virtual steps.
hipError_t chunk_split_dispatch(int64_t BH, int64_t T, int nh, int dk, int dv, const void* q, const void* k,
                                const void* v, const float* g, const float* beta, const float* S0, void* o, float* Sf,
                                void* ws, hipStream_t st) {
    const int64_t Tv = T * nh;
    const int64_t nC = (Tv + kChunk - 1) / kChunk;
    const uint32_t magic = nh > 1 ? (uint32_t)(((uint64_t(1) << 32) + nh - 1) / nh) : 0u;
    UtArgs u;
    u.H = 1;
    u.A_log = nullptr;
    u.dt_bias = nullptr;
    u.T = Tv;
    u.Treal = T;
    u.nh = (uint32_t)nh;
    u.nh_magic = magic;
    u.nC = nC;
    u.q = static_cast<const uint16_t*>(q);
    u.k = static_cast<const uint16_t*>(k);
    u.g = g;
    u.beta = beta;
    u.ws = static_cast<uint16_t*>(ws);
    StArgs s;
    s.T = Tv;
    s.Treal = T;
    s.nh = (uint32_t)nh;
    s.nh_magic = magic;
    s.nC = nC;
    s.dv = dv;
    s.ntiles = dv / 32;
    s.q = u.q;
    s.k = u.k;
    s.v = static_cast<const uint16_t*>(v);
    s.wg = nullptr;
    s.ws = u.ws;
    s.S0 = S0;
    s.o = static_cast<uint16_t*>(o);
    s.Sf = Sf;
    if (nh > 1) {
        if (dk == 128) return launch_split<128, kUtVirt>(u, s, BH, st);
        return launch_split<64, kUtVirt>(u, s, BH, st);
    }
    if (dk == 128) return launch_split<128, kUtPlain>(u, s, BH, st);
    return launch_split<64, kUtPlain>(u, s, BH, st);
}

// Bytes of workspace of the two-kernel path with fused input preparation: 13120 per (sequence,
// chunk) for either dk.
int64_t chunk_split_prep_workspace_bytes(int64_t BH, int64_t T, int dk) {
    (void)dk;
    const int64_t nC = (T + kChunk - 1) / kChunk;
    return BH * nC * kPrepWsStride * 2;
}

// Gated DeltaNet from raw projections on the two-kernel path: q_raw, k_raw [BH][T][dk] bf16,
// dt and beta_logit [BH][T], A_log and dt_bias [H] (bh mod H is the head).
hipError_t chunk_split_prep_dispatch(int64_t BH, int64_t H, int64_t T, int dk, int dv, const void* q_raw,
                                     const void* k_raw, const void* v, const float* dt, const float* A_log,
                                     const float* dt_bias, const float* beta_logit, const float* S0, void* o,
                                     float* Sf, void* ws, hipStream_t st) {
    const int64_t nC = (T + kChunk - 1) / kChunk;
    UtArgs u;
    u.H = (int)H;
    u.A_log = A_log;
    u.dt_bias = dt_bias;
    u.T = T;
    u.Treal = T;
    u.nh = 1;
    u.nh_magic = 0u;
    u.nC = nC;
    u.q = static_cast<const uint16_t*>(q_raw);
    u.k = static_cast<const uint16_t*>(k_raw);
    u.g = dt;
    u.beta = beta_logit;
    u.ws = static_cast<uint16_t*>(ws);
    StArgs s;
    s.T = T;
    s.Treal = T;
    s.nh = 1;
    s.nh_magic = 0u;
    s.nC = nC;
    s.dv = dv;
    s.ntiles = dv / 32;
    s.q = u.q;
    s.k = u.k;
    s.v = static_cast<const uint16_t*>(v);
    s.wg = nullptr;
    s.ws = u.ws;
    s.S0 = S0;
    s.o = static_cast<uint16_t*>(o);
    s.Sf = Sf;
    if (dk == 128) return launch_split<128, kUtPrep>(u, s, BH, st);
    return launch_split<64, kUtPrep>(u, s, BH, st);
}

// State pass of the per-channel-gate two-kernel path, over a workspace the KDA UT pass has
// filled (chunk_kda_ut_dispatch): kda_ws_stride<dk>() halfs per (sequence, chunk).
hipError_t chunk_state_kda_dispatch(int64_t BH, int64_t T, int dk, int dv, const void* v, const float* wg,
                                    const float* S0, void* o, float* Sf, const void* ws, hipStream_t st) {
    StArgs s;
    s.T = T;
    s.Treal = T;
    s.nh = 1;
    s.nh_magic = 0u;
    s.nC = (T + kChunk - 1) / kChunk;
    s.dv = dv;
    s.ntiles = dv / 32;
    s.q = nullptr;
    s.k = nullptr;
    s.v = static_cast<const uint16_t*>(v);
    s.wg = wg;
    s.ws = static_cast<const uint16_t*>(ws);
    s.S0 = S0;
    s.o = static_cast<uint16_t*>(o);
    s.Sf = Sf;
    if (wg) {
        if (dk == 128) return launch_state<128, kStGd2>(s, BH, st);
        return launch_state<64, kStGd2>(s, BH, st);
    }
    if (dk == 128) return launch_state<128, kStKda>(s, BH, st);
    return launch_state<64, kStKda>(s, BH, st);
}

}  // namespace gdr
