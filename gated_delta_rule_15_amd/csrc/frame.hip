// frame.hip -- the frame-level implicit delta-rule update, bf16 I/O, gfx950.
//
// The video delta-rule post (haoyizhu.site, "video-delta-rule"), section "A Different Route":
// tokens come in frames of n with no order inside a frame, and one frame moves the state by
// one implicit (backward-Euler) gradient step on the frame's total loss.  Column convention,
// S in R^{d_v x d_k}:
//   G_t = K_t^T Gamma_t K_t,   C_t = V_t^T Gamma_t K_t,   S_t (I + G_t) = S_{t-1} D_t + C_t,
//   o_{t,i} = S_t q_{t,i}  for every token of frame t,
// with Gamma_t the per-token writing strengths and D_t the frame's forget gate (scalar or per
// key channel) applied to the old state first.  I + G_t does not depend on the state, so
// everything but one product per frame runs for all frames at once:
//
//   frame_gram_kernel   one workgroup per (sequence, frame): G and C by fp16 MFMA over the
//                       frame's tokens (operands sqrt(gamma) k and sqrt(gamma) v, fp32
//                       accumulation), then W = (I + G)^{-1} by blocked in-place Gauss-Jordan
//                       elimination in fp32 (16 x 16 pivot blocks inverted in registers, the
//                       panels and rank-16 updates on fp32 MFMA; I + G is symmetric positive
//                       definite with eigenvalues >= 1, so no pivoting is needed), written as a
//                       pair of fp16 matrices W = W_hi + W_lo, and C in fp32;
//   frame_state_kernel  one workgroup per (sequence, 32 value channels), frames in order:
//                       S_t^T = W_t (D_t S_{t-1}^T + C_t^T) on fp16 MFMA with both factors split
//                       into high and low halves (three products: hi.hi + hi.lo + lo.hi), which
//                       keeps the chained state at fp32-class accuracy; S_t is written in fp16
//                       for the outputs;
//   frame_out_kernel    one workgroup per (sequence, 512 tokens): O = Q S_t^T.
// The post solves the system by a Cholesky factorisation; forming the inverse once per frame
// instead keeps the serial pass to one product per frame (the same solution in exact
// arithmetic; I + G is never singular, its eigenvalues lying in [1, 1 + tr G]).
#include "chunk_common.h"

namespace gdr {

struct FrArgs {
    int64_t T;
    int64_t F;       // frames per sequence, ceil(T / n)
    int n;           // tokens per frame (a multiple of 16)
    int channel;     // gate per key channel (1) or scalar (0)
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* gamma;
    const float* g;  // log forget gate, [.., F] or [.., F, DK]
    const float* S0;
    uint16_t* o;
    float* Sf;
    // workspace, per (sequence, frame): W_hi, W_lo [DK][DK] fp16, C [DV][DK] fp32, S [DV][DK] fp16
    uint16_t* Wh;
    uint16_t* Wl;
    float* Cw;
    uint16_t* Sw;
    int* Ew;         // per (sequence, frame, 16 value channels): the power of two Sw is scaled by
};

// ============================================================================ Gram + inverse

template <int DK, int DV>
struct FrGramLds {
    static constexpr int LDK = DK + 16;   // halfs, token rows of sqrt(gamma) k
    static constexpr int LDV = DV + 16;   // halfs, token rows of sqrt(gamma) v
    static constexpr int LDA = DK + 4;    // floats, rows of I + G
    static constexpr int szK = 64 * LDK * 2, szV = 64 * LDV * 2;
    static constexpr int oK = 0;                // two buffers each
    static constexpr int oV = oK + 2 * szK;
    static constexpr int oA = oV + 2 * szV;
    static constexpr int total = oA + DK * LDA * 4;
    static_assert(total <= 160 * 1024, "LDS budget");
};

template <int DK, int DV>
__global__ __launch_bounds__(256, 1) void frame_gram_kernel(const FrArgs a) {
    using L = FrGramLds<DK, DV>;
    constexpr int NT = DK / 16, NV = DV / 16;
    constexpr int NSG = (NT + 3) / 4, NSC = (NV + 3) / 4;  // row tiles per wave
    extern __shared__ __attribute__((aligned(16))) char smem[];
    auto Kbuf = [&](int b) { return reinterpret_cast<_Float16*>(smem + L::oK + b * L::szK); };
    auto Vbuf = [&](int b) { return reinterpret_cast<_Float16*>(smem + L::oV + b * L::szV); };
    float* Am = reinterpret_cast<float*>(smem + L::oA);

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, j = l & 15, g = l >> 4;
    const int64_t bh = blockIdx.x / a.F;
    const int64_t f = blockIdx.x - bh * a.F;
    const int64_t T = a.T;
    const int64_t t_beg = f * a.n;
    const int64_t t_end = (t_beg + a.n < T) ? t_beg + a.n : T;
    const auto rk = make_rsrc(a.k + bh * T * DK, (uint32_t)(T * DK * 2));
    const auto rv = make_rsrc(a.v + bh * T * DV, (uint32_t)(T * DV * 2));
    const auto rgm = make_rsrc(a.gamma + bh * T, (uint32_t)(T * 4));

    auto trfrag = [&](const _Float16* base, int ld, int kb, int col) {
        const _Float16* p0 = base + (32 * kb + 4 * g + (j >> 2)) * ld + col;
        return cat8(ldtr(p0), ldtr(p0 + 16 * ld));
    };

    // accumulators: G row tiles ti = w + 4s (tiles tj <= ti), C row tiles vi = w + 4s
    float4v accG[NSG][NT], accC[NSC][NT];
#pragma unroll
    for (int s = 0; s < NSG; ++s)
#pragma unroll
        for (int t = 0; t < NT; ++t) accG[s][t] = zero4();
#pragma unroll
    for (int s = 0; s < NSC; ++s)
#pragma unroll
        for (int t = 0; t < NT; ++t) accC[s][t] = zero4();

    // ---- G and C over the frame's tokens, 64 at a time.  Thread tid stages the 16-byte pieces
    // (row, col) with row = tid / R + (256 / R) i of K (R = DK / 8 pieces per row) and of V
    // (R = DV / 8); a block's pieces, and in each wave the gamma of the block's 64 tokens (one
    // per lane), are loaded into registers two blocks before it is staged.  Tokens outside the
    // frame read past the buffer end, which returns zeros.
    constexpr int RK = DK / 8, RV = DV / 8, NPK = 64 * RK / 256, NPV = 64 * RV / 256;
    struct Blk {
        uint4 kp[NPK], vp[NPV];
        float gm;  // gamma of the block's token l (every wave loads the block's 64)
    };
    Blk B0, B1;  // blocks alternate between the two register sets
    auto load_block = [&](Blk& B, int64_t t0) {
#pragma unroll
        for (int i = 0; i < NPK; ++i) {
            const int row = tid / RK + (256 / RK) * i, col = (tid % RK) * 8;
            const int64_t tok = t0 + row;
            const bool in = tok < t_end;
            B.kp[i] = bld16(rk, in ? (uint32_t)((tok * DK + col) * 2) : (uint32_t)(T * DK * 2));
        }
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
            const int row = tid / RV + (256 / RV) * i, col = (tid % RV) * 8;
            const int64_t tok = t0 + row;
            const bool in = tok < t_end;
            B.vp[i] = bld16(rv, in ? (uint32_t)((tok * DV + col) * 2) : (uint32_t)(T * DV * 2));
        }
        B.gm = bld4(rgm, t0 + l < t_end ? (uint32_t)((t0 + l) * 4) : (uint32_t)(T * 4));
    };
    auto scaled = [](const uint4& u, float sg) {
        const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
        half8 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            h[2 * e] = (_Float16)(sg * __uint_as_float(wv[e] << 16));
            h[2 * e + 1] = (_Float16)(sg * __uint_as_float(wv[e] & 0xffff0000u));
        }
        return h;
    };
    // a row's sqrt(gamma) comes from the lane that loaded its gamma (ds_bpermute)
    auto stage_block = [&](const Blk& B, _Float16* Kp, _Float16* Vp) {
        const int sgl = __float_as_int(sqrtf(B.gm));
#pragma unroll
        for (int i = 0; i < NPK; ++i) {
            const int row = tid / RK + (256 / RK) * i, col = (tid % RK) * 8;
            const float sg = __int_as_float(__builtin_amdgcn_ds_bpermute(row * 4, sgl));
            *reinterpret_cast<half8*>(Kp + row * L::LDK + col) = scaled(B.kp[i], sg);
        }
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
            const int row = tid / RV + (256 / RV) * i, col = (tid % RV) * 8;
            const float sg = __int_as_float(__builtin_amdgcn_ds_bpermute(row * 4, sgl));
            *reinterpret_cast<half8*>(Vp + row * L::LDV + col) = scaled(B.vp[i], sg);
        }
    };
    // the products of one staged block
    auto products = [&](const _Float16* Kp, const _Float16* Vp) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            half8 kf[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) kf[t] = trfrag(Kp, L::LDK, kb, 16 * t + 4 * (j & 3));
#pragma unroll
            for (int s = 0; s < NSG; ++s) {
                const int ti = w + 4 * s;
                if (ti < NT) {
                    const half8 kr = trfrag(Kp, L::LDK, kb, 16 * ti + 4 * (j & 3));
#pragma unroll
                    for (int tj = 0; tj < NT; ++tj)
                        if (tj <= ti) mma16(accG[s][tj], kr, kf[tj]);
                }
            }
#pragma unroll
            for (int s = 0; s < NSC; ++s) {
                const int vi = w + 4 * s;
                if (vi < NV) {
                    const half8 vr = trfrag(Vp, L::LDV, kb, 16 * vi + 4 * (j & 3));
#pragma unroll
                    for (int tj = 0; tj < NT; ++tj) mma16(accC[s][tj], vr, kf[tj]);
                }
            }
        }
    };
    // one step: stage the next block (register set Bn) into LDS buffer bn, refill Bn with the
    // block three ahead (past the frame: zeros, no memory traffic, and no branch, so that the
    // other set's loads stay in flight), then the products of the block in buffer 1 - bn.  One
    // barrier per block: the buffer being staged was last read by the step before.
    auto step = [&](Blk& Bn, int bn, int64_t t_refill) {
        stage_block(Bn, Kbuf(bn), Vbuf(bn));
        load_block(Bn, t_refill);
        products(Kbuf(1 - bn), Vbuf(1 - bn));
        lds_barrier();
    };
    load_block(B0, t_beg);
    load_block(B1, t_beg + 64);
    stage_block(B0, Kbuf(0), Vbuf(0));
    load_block(B0, t_beg + 128);
    lds_barrier();
    int64_t t0 = t_beg;
    for (; t0 + 64 < t_end; t0 += 128) {
        step(B1, 1, t0 + 192);  // products of the block at t0 (buffer 0)
        step(B0, 0, t0 + 256);  // products of the block at t0 + 64 (buffer 1)
    }
    if (t0 < t_end) step(B1, 1, t0 + 192);

    // ---- I + G into LDS (both triangles), C to the workspace
    const int64_t fi = bh * a.F + f;
#pragma unroll
    for (int s = 0; s < NSG; ++s) {
        const int ti = w + 4 * s;
        if (ti < NT) {
#pragma unroll
            for (int tj = 0; tj < NT; ++tj) {
                if (tj <= ti) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = 16 * ti + 4 * g + r, col = 16 * tj + j;
                        const float x = accG[s][tj][r] + (row == col ? 1.0f : 0.0f);
                        Am[row * L::LDA + col] = x;
                        Am[col * L::LDA + row] = x;
                    }
                }
            }
        }
    }
    float* cdst = a.Cw + fi * (int64_t)(DV * DK);
#pragma unroll
    for (int s = 0; s < NSC; ++s) {
        const int vi = w + 4 * s;
        if (vi < NV) {
#pragma unroll
            for (int tj = 0; tj < NT; ++tj)
#pragma unroll
                for (int r = 0; r < 4; ++r) cdst[(16 * vi + 4 * g + r) * DK + 16 * tj + j] = accC[s][tj][r];
        }
    }
    lds_barrier();

    // ---- W = (I + G)^{-1} by blocked Gauss-Jordan elimination in place, 16 pivots per block.
    // For pivot block K (rows and columns Kb = 16K .. 16K + 15):
    //   1. wave 0 inverts the 16 x 16 pivot tile D = A_{Kb,Kb} alone by Gauss-Jordan (fp32
    //      registers, four entries per lane);
    //   2. the panel: the other rows of column block K become P_i = -A_{i,Kb} D^{-1} (fp32
    //      MFMA, 16x16x4);
    //   3. every other column block j takes the 16 pivots at once as a rank-16 product,
    //      A_ij <- A_ij + P_i A_{Kb,j} (i != K) and A_{Kb,j} <- D^{-1} A_{Kb,j}, every tile read
    //      before any is written.
    // This is the pivot-by-pivot elimination regrouped (the same operations in exact
    // arithmetic): the panel sees its 16 pivots one by one, the rest of the matrix sees their
    // product.  I + G is symmetric positive definite with eigenvalues >= 1, and so is every
    // pivot block's Schur complement: no pivoting is needed.  Steps 2 and 3 are split by row
    // blocks: wave w owns row blocks w, w + 4, .. and forms their panel tiles and then their
    // trailing tiles, so that a row's P_i fragments are read once for its tiles and the row
    // block K fragments once for all of a wave's rows, and no barrier separates the panel from
    // the update (a wave reads only its own rows of column block K).
    constexpr int NB = DK / 16;          // pivot blocks
    constexpr int NRW = NB / 4;          // row blocks per wave
    static_assert(NB % 4 == 0, "every wave owns whole row blocks");
    for (int kbk = 0; kbk < NB; ++kbk) {
        const int kc = 16 * kbk;
        // 1. wave 0: D^{-1}.  Lane (r, cg) = (l % 16, l / 16) holds row r, columns 4cg .. 4cg + 3;
        //    for pivot p it fetches row p's four entries of its columns and its own row's
        //    column-p entry from the lanes that hold them (ds_bpermute), the pivot by readlane
        if (w == 0) {
            const int r = l & 15, cg = l >> 4;
            float4v x = ld4f(Am + (kc + r) * L::LDA + kc + 4 * cg);
#pragma unroll
            for (int pp = 0; pp < 16; ++pp) {
                const int src_p = (16 * cg + pp) * 4;               // row pp, this column group
                const int src_f = (16 * (pp >> 2) + r) * 4;         // row r, column pp
                float rowp[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) rowp[e] = __int_as_float(__builtin_amdgcn_ds_bpermute(src_p, __float_as_int(x[e])));
                const float f = __int_as_float(__builtin_amdgcn_ds_bpermute(src_f, __float_as_int(x[pp & 3])));
                const float dp = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x[pp & 3]), 16 * (pp >> 2) + pp));
                const float rp = __builtin_amdgcn_rcpf(dp);  // 1 ulp; the pivots are >= 1 in exact arithmetic
                const bool prow = r == pp;
                const float keep = prow ? 0.0f : 1.0f;
                const float cf = prow ? rp : -f * rp;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = fmaf(rowp[e], cf, x[e] * keep);
                if (cg == (pp >> 2)) x[pp & 3] = prow ? rp : -f * rp;
            }
            *reinterpret_cast<float4v*>(Am + (kc + r) * L::LDA + kc + 4 * cg) = x;
        }
        lds_barrier();
        // 2. this wave's panel tiles (row blocks ib = w + 4u other than K), written in place
#pragma unroll
        for (int u = 0; u < NRW; ++u) {
            const int ib = w + 4 * u;
            if (ib != kbk) {
                float4v a4 = zero4();
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float av = Am[(16 * ib + j) * L::LDA + kc + 4 * q + g];  // A[16 ib + j][Kb + 4q + g]
                    const float bv = Am[(kc + 4 * q + g) * L::LDA + kc + j];       // D^{-1}[4q + g][j]
                    a4 = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, a4, 0, 0, 0);
                }
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) Am[(16 * ib + 4 * g + r4) * L::LDA + kc + j] = -a4[r4];
            }
        }
        lds_fence();  // this wave's panel stores before it reads them back as operands
        // 3. this wave's trailing tiles: P fragments of its rows (row block K: D^{-1}), then
        //    each column block jb != K with its row block K fragments
        float pa[NRW][4];
#pragma unroll
        for (int u = 0; u < NRW; ++u) {
            const int ib = w + 4 * u;
#pragma unroll
            for (int q = 0; q < 4; ++q) pa[u][q] = Am[(16 * ib + j) * L::LDA + kc + 4 * q + g];  // P[16 ib + j][4q + g]
        }
        // (no branch in the loop, so that the next column's loads can go out under the current
        // column's products: row block K loads its old tile too and starts from zero instead)
        float4v acc[NRW][NB - 1];
#pragma unroll
        for (int jr = 0; jr < NB - 1; ++jr) {
            const int jb = jr + (jr >= kbk ? 1 : 0);
            float pb[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) pb[q] = Am[(kc + 4 * q + g) * L::LDA + 16 * jb + j];  // A[Kb + 4q + g][16 jb + j]
#pragma unroll
            for (int u = 0; u < NRW; ++u) {
                const int ib = w + 4 * u;
                float4v a4;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float old = Am[(16 * ib + 4 * g + r) * L::LDA + 16 * jb + j];
                    a4[r] = ib != kbk ? old : 0.0f;
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) a4 = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[u][q], pb[q], a4, 0, 0, 0);
                acc[u][jr] = a4;
            }
        }
        lds_barrier();
#pragma unroll
        for (int u = 0; u < NRW; ++u) {
            const int ib = w + 4 * u;
#pragma unroll
            for (int jr = 0; jr < NB - 1; ++jr) {
                const int jb = jr + (jr >= kbk ? 1 : 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) Am[(16 * ib + 4 * g + r) * L::LDA + 16 * jb + j] = acc[u][jr][r];
            }
        }
        lds_barrier();
    }
    // W as W_hi + W_lo (fp16 each), rows natural, in pieces of 8 columns: consecutive threads
    // take consecutive pieces of a row (conflict-free LDS reads, 16-byte stores)
    constexpr int PPR = DK / 8, NPW = DK * PPR / 256;
    uint16_t* wh = a.Wh + fi * (int64_t)(DK * DK);
    uint16_t* wl = a.Wl + fi * (int64_t)(DK * DK);
#pragma unroll
    for (int u = 0; u < NPW; ++u) {
        const int idx = tid + 256 * u, row = idx / PPR, col = (idx % PPR) * 8;
        const float4v x0 = ld4f(Am + row * L::LDA + col), x1 = ld4f(Am + row * L::LDA + col + 4);
        half8 hh, hl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float xv = e < 4 ? x0[e] : x1[e - 4];
            hh[e] = (_Float16)xv;
            hl[e] = (_Float16)(xv - (float)hh[e]);
        }
        *reinterpret_cast<half8*>(wh + row * DK + col) = hh;
        *reinterpret_cast<half8*>(wl + row * DK + col) = hl;
    }
}

// ============================================================================ state pass

template <int DK>
struct FrStateLds {
    static constexpr int LDW = DK + 8;  // halfs, rows of W_hi / W_lo
    static constexpr int oWh = 0;
    static constexpr int oWl = oWh + DK * LDW * 2;
    static constexpr int total = oWl + DK * LDW * 2;
};

template <int DK, int DV, int NWV, bool CH>
__global__ __launch_bounds__(64 * NWV, 1) void frame_state_kernel(const FrArgs a) {
    using L = FrStateLds<DK>;
    constexpr int NKB = DK / 32, NST = DK / 16;
    constexpr int NTH = 64 * NWV;           // threads: NWV waves of 16 value channels
    constexpr int NPW = DK * DK / 8 / NTH;  // 16-byte pieces of one W matrix per thread
    extern __shared__ __attribute__((aligned(16))) char smem[];
    _Float16* Whs = reinterpret_cast<_Float16*>(smem + L::oWh);
    _Float16* Wls = reinterpret_cast<_Float16*>(smem + L::oWl);

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, j = l & 15, g = l >> 4;
    constexpr int NDT = DV / (16 * NWV);  // workgroups per sequence
    const int64_t bh = blockIdx.x / NDT;
    const int dvc = (int)(blockIdx.x % NDT) * (16 * NWV) + 16 * w;  // this wave's first value channel
    const int64_t F = a.F;

    // S^T of 16 value channels, rows permuted by pperm (row P holds key channel pperm(P))
    float4v St[NST];
#pragma unroll
    for (int t = 0; t < NST; ++t) St[t] = zero4();
    if (a.S0 != nullptr) {
        const float* s0 = a.S0 + bh * (int64_t)DV * DK + (int64_t)(dvc + j) * DK;
#pragma unroll
        for (int t = 0; t < NST; ++t) St[t] = ld4f(s0 + pperm(16 * t + 4 * g));
    }

    // W of the next frame, prefetched into registers one frame ahead (buffer loads: the
    // offsets stay below 2^31 per sequence)
    const auto rwh = make_rsrc(a.Wh + bh * F * (int64_t)(DK * DK), (uint32_t)(F * DK * DK * 2));
    const auto rwl = make_rsrc(a.Wl + bh * F * (int64_t)(DK * DK), (uint32_t)(F * DK * DK * 2));
    uint4 wph[NPW], wpl[NPW];
#pragma unroll
    for (int u = 0; u < NPW; ++u) {
        wph[u] = bld16(rwh, (uint32_t)((tid + NTH * u) * 16));
        wpl[u] = bld16(rwl, (uint32_t)((tid + NTH * u) * 16));
    }
    // C and the frame gate of the next frame, prefetched the same way (buffer loads, no branch:
    // past the last frame they read zeros, which are never used).  The scalar gate is one dword
    // per frame.
    constexpr int gstride = CH ? DK : 1;
    const auto rc = make_rsrc(a.Cw + bh * F * (int64_t)(DV * DK), (uint32_t)(F * DV * DK * 4));
    const auto rgf = make_rsrc(a.g + bh * F * gstride, (uint32_t)(F * gstride * 4));
    float4v cn[NST], gn[CH ? NST : 1];
    auto load_cg = [&](int64_t fl) {
#pragma unroll
        for (int t = 0; t < NST; ++t) {
            const int ch = pperm(16 * t + 4 * g);
            cn[t] = __builtin_bit_cast(float4v, bld16(rc, (uint32_t)(((fl * DV + dvc + j) * DK + ch) * 4)));
            if constexpr (CH) gn[t] = __builtin_bit_cast(float4v, bld16(rgf, (uint32_t)((fl * DK + ch) * 4)));
        }
        if constexpr (!CH) gn[0][0] = bld4(rgf, (uint32_t)(fl * 4));
    };
    load_cg(0);
    for (int64_t f = 0; f < F; ++f) {
        const int64_t fi = bh * F + f;
        // rhs^T = D S^T + C^T (rows permuted as S^T), then the next frame's C and gate
        float4v rh[NST];
#pragma unroll
        for (int t = 0; t < NST; ++t) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float d = fast_exp(CH ? gn[t][r] : gn[0][0]);
                rh[t][r] = fmaf(d, St[t][r], cn[t][r]);
            }
        }
        // rhs is split into fp16 halves below; a power of two per wave brings its largest
        // magnitude near 2^12 first (C grows with the writing strength and the frame length
        // even when the state does not), and the product is scaled back after it
        int rexp = 0;
        {
            const float M = wave_max_abs(max_abs(rh));
            if (M > 0.0f && M <= 3.0e38f) rexp = min(max(12 - __builtin_amdgcn_frexp_expf(M), -100), 100);
            const float sc = __builtin_ldexpf(1.0f, rexp);
#pragma unroll
            for (int t = 0; t < NST; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) rh[t][r] *= sc;
        }
        load_cg(f + 1);
        // W of this frame into LDS (the previous frame's readers are past the barrier below)
#pragma unroll
        for (int u = 0; u < NPW; ++u) {
            const int idx = tid + NTH * u, row = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            *reinterpret_cast<uint4*>(Whs + row * L::LDW + col) = wph[u];
            *reinterpret_cast<uint4*>(Wls + row * L::LDW + col) = wpl[u];
        }
        lds_barrier();
        // operand halves: rhs = hi + lo
        half8 bh8[NKB], bl8[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            bh8[kb] = pack8(rh[2 * kb], rh[2 * kb + 1]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float full = e < 4 ? rh[2 * kb][e] : rh[2 * kb + 1][e - 4];
                bl8[kb][e] = (_Float16)(full - (float)bh8[kb][e]);
            }
        }
        // S^T = W rhs^T: row tile t uses W rows pperm(16 t + j), 8 consecutive key channels.  Two
        // tiles at a time, so that two accumulation chains interleave; after each pair the
        // registers W was staged from take the next frame's W pieces a few at a time (past the
        // end: zeros, unused), so that their issue overlaps the products.
        static_assert(NST % 2 == 0 && NPW % (NST / 2) == 0, "W pieces per tile pair");
        constexpr int LPP = NPW / (NST / 2);
        const uint32_t nb = (uint32_t)((f + 1) * DK * DK * 2);
        const float isc = __builtin_ldexpf(1.0f, -rexp);
#pragma unroll
        for (int t = 0; t < NST; t += 2) {
            float4v acc0 = zero4(), acc1 = zero4();
            const int wr0 = pperm(16 * t + j), wr1 = pperm(16 * (t + 1) + j);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const half8 ah0 = ld8(Whs + wr0 * L::LDW + 32 * kb + 8 * g);
                const half8 al0 = ld8(Wls + wr0 * L::LDW + 32 * kb + 8 * g);
                const half8 ah1 = ld8(Whs + wr1 * L::LDW + 32 * kb + 8 * g);
                const half8 al1 = ld8(Wls + wr1 * L::LDW + 32 * kb + 8 * g);
                mma16(acc0, ah0, bh8[kb]);
                mma16(acc1, ah1, bh8[kb]);
                mma16(acc0, ah0, bl8[kb]);
                mma16(acc1, ah1, bl8[kb]);
                mma16(acc0, al0, bh8[kb]);
                mma16(acc1, al1, bh8[kb]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                St[t][r] = acc0[r] * isc;
                St[t + 1][r] = acc1[r] * isc;
            }
#pragma unroll
            for (int u = (t / 2) * LPP; u < (t / 2 + 1) * LPP; ++u) {
                wph[u] = bld16(rwh, nb + (uint32_t)((tid + NTH * u) * 16));
                wpl[u] = bld16(rwl, nb + (uint32_t)((tid + NTH * u) * 16));
            }
        }
        // S_t in fp16, [value channel][key channel], for the outputs, times a power of two per
        // wave that brings its largest magnitude near 2^12 (stored beside it for the outputs)
        {
            const float M = wave_max_abs(max_abs(St));
            int sexp = 0;
            if (M > 0.0f && M <= 3.0e38f) sexp = min(max(12 - __builtin_amdgcn_frexp_expf(M), -100), 100);
            const float sc = __builtin_ldexpf(1.0f, sexp);
            uint16_t* sd = a.Sw + fi * (int64_t)(DV * DK) + (int64_t)(dvc + j) * DK;
#pragma unroll
            for (int t = 0; t < NST; ++t) {
                const half4 h = half4{(_Float16)(St[t][0] * sc), (_Float16)(St[t][1] * sc), (_Float16)(St[t][2] * sc),
                                      (_Float16)(St[t][3] * sc)};
                *reinterpret_cast<half4*>(sd + pperm(16 * t + 4 * g)) = h;
            }
            if (l == 0) a.Ew[fi * (DV / 16) + dvc / 16] = sexp;
        }
        lds_barrier();
    }
    if (a.Sf != nullptr) {
        float* sf = a.Sf + bh * (int64_t)DV * DK + (int64_t)(dvc + j) * DK;
#pragma unroll
        for (int t = 0; t < NST; ++t) *reinterpret_cast<float4v*>(sf + pperm(16 * t + 4 * g)) = St[t];
    }
}

// ============================================================================ outputs

template <int DV>
struct FrOutLds {
    static constexpr int LDO = DV + 8;  // bf16, token rows of the output tile
    static constexpr int total = 64 * LDO * 2;
};

// One group per 512 tokens of a sequence; wave w takes tokens 128 w .. 128 w + 127 of them in
// eight 16-token steps.  The frame state's operand fragments (all of S_t^T, fp16) stay in the
// wave's registers and are reloaded only when a step enters a new frame, so each wave reads S
// once for up to 128 tokens instead of once per 16.
template <int DK, int DV>
__global__ __launch_bounds__(256) void frame_out_kernel(const FrArgs a, int64_t nblk) {
    using L = FrOutLds<DV>;
    constexpr int NKB = DK / 32, NV = DV / 16, NG = 8;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    uint16_t* Ot = reinterpret_cast<uint16_t*>(smem);
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, j = l & 15, g = l >> 4;
    const int64_t bh = blockIdx.x / nblk;
    const int64_t blk = blockIdx.x - bh * nblk;
    const int64_t T = a.T;
    const auto rq = make_rsrc(a.q + bh * T * DK, (uint32_t)(T * DK * 2));
    const auto ro = make_rsrc(a.o + bh * T * DV, (uint32_t)(T * DV * 2));
    half8 sf[NV][NKB];
    float osc[NV];  // 2^-exponent of each 16-channel group of the frame's state copy
    int64_t fcur = -1;
    for (int gi = 0; gi < NG; ++gi) {
        const int64_t tb = blk * 512 + 128 * w + 16 * gi;  // this step's 16 tokens, all in one frame
        if (tb >= T) break;
        const int64_t f = tb / a.n;
        if (f != fcur) {
            const uint16_t* S = a.Sw + (bh * a.F + f) * (int64_t)(DV * DK);
#pragma unroll
            for (int vi = 0; vi < NV; ++vi) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
                    sf[vi][kb] = *reinterpret_cast<const half8*>(S + (16 * vi + j) * DK + 32 * kb + 8 * g);
                osc[vi] = __builtin_ldexpf(1.0f, -a.Ew[(bh * a.F + f) * NV + vi]);
            }
            fcur = f;
        }
        half8 qa[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
            qa[kb] = bf16x8_to_half8(bld16(rq, (uint32_t)(((tb + j) * DK + 32 * kb + 8 * g) * 2)));
#pragma unroll
        for (int vi = 0; vi < NV; ++vi) {
            float4v acc = zero4();
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) mma16(acc, qa[kb], sf[vi][kb]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t b2 = pack_bf16x2(acc[r] * osc[vi], 0.0f);
                Ot[(16 * w + 4 * g + r) * L::LDO + 16 * vi + j] = (uint16_t)(b2 & 0xffffu);
            }
        }
        lds_fence();
        // this wave's 16 token rows back as 16-byte pieces (rows past the end are dropped)
        constexpr int PPR = DV / 8;  // pieces per row
#pragma unroll
        for (int u = 0; u < 16 * PPR / 64; ++u) {
            const int idx = l + 64 * u, row = idx / PPR, col = (idx % PPR) * 8;
            const uint4 val = *reinterpret_cast<const uint4*>(Ot + (16 * w + row) * L::LDO + col);
            bst16(ro, (uint32_t)(((tb + row) * DV + col) * 2), val);
        }
        lds_fence();  // the next step rewrites these rows
    }
}

// ============================================================================ host side

int64_t frame_workspace_bytes(int64_t BH, int64_t T, int n, int dk, int dv) {
    const int64_t F = (T + n - 1) / n;
    return BH * F * ((int64_t)dk * dk * 2 * 2 + (int64_t)dv * dk * 4 + (int64_t)dv * dk * 2 + (int64_t)dv / 16 * 4);
}

template <int DK, int DV>
static hipError_t launch_frame(const FrArgs& a, int64_t BH, hipStream_t st) {
    constexpr int lds_gram = FrGramLds<DK, DV>::total, lds_state = FrStateLds<DK>::total;
    constexpr int lds_out = FrOutLds<DV>::total;
    static std::atomic<uint64_t> lds_enabled{0};  // one bit per device
    if (const hipError_t e = enable_dynamic_lds(frame_gram_kernel<DK, DV>, lds_gram, lds_enabled); e != hipSuccess)
        return e;
    if (a.F > 0) {
        hipLaunchKernelGGL((frame_gram_kernel<DK, DV>), dim3((unsigned)(BH * a.F)), dim3(256), lds_gram, st, a);
    }
    constexpr int kStateWaves = 2;  // value-channel tiles of 32: more groups, each reading W once
    if (a.channel)
        hipLaunchKernelGGL((frame_state_kernel<DK, DV, kStateWaves, true>), dim3((unsigned)(BH * (DV / (16 * kStateWaves)))),
                           dim3(64 * kStateWaves), lds_state, st, a);
    else
        hipLaunchKernelGGL((frame_state_kernel<DK, DV, kStateWaves, false>),
                           dim3((unsigned)(BH * (DV / (16 * kStateWaves)))), dim3(64 * kStateWaves), lds_state, st, a);
    const int64_t nblk = (a.T + 511) / 512;
    if (nblk > 0) {
        hipLaunchKernelGGL((frame_out_kernel<DK, DV>), dim3((unsigned)(BH * nblk)), dim3(256), lds_out, st, a,
                           nblk);
    }
    return hipGetLastError();
}

hipError_t frame_dispatch(int64_t BH, int64_t T, int n, int dk, int dv, bool channel, const void* q, const void* k,
                          const void* v, const float* gamma, const float* g, const float* S0, void* o, float* Sf,
                          void* ws, hipStream_t st) {
    FrArgs a;
    a.T = T;
    a.F = (T + n - 1) / n;
    a.n = n;
    a.channel = channel ? 1 : 0;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.gamma = gamma;
    a.g = g;
    a.S0 = S0;
    a.o = static_cast<uint16_t*>(o);
    a.Sf = Sf;
    const int64_t nf = BH * a.F;
    char* base = static_cast<char*>(ws);
    a.Wh = reinterpret_cast<uint16_t*>(base);
    a.Wl = reinterpret_cast<uint16_t*>(base + nf * (int64_t)dk * dk * 2);
    a.Cw = reinterpret_cast<float*>(base + nf * (int64_t)dk * dk * 4);
    a.Sw = reinterpret_cast<uint16_t*>(base + nf * ((int64_t)dk * dk * 4 + (int64_t)dv * dk * 4));
    a.Ew = reinterpret_cast<int*>(base + nf * ((int64_t)dk * dk * 4 + (int64_t)dv * dk * 6));
    if (dk == 128 && dv == 128) return launch_frame<128, 128>(a, BH, st);
    if (dk == 128 && dv == 64) return launch_frame<128, 64>(a, BH, st);
    if (dk == 64 && dv == 128) return launch_frame<64, 128>(a, BH, st);
    return launch_frame<64, 64>(a, BH, st);
}

}  // namespace gdr
