// chunk_fwd_pc.hip -- producer/consumer chunked forward of the gated delta rule (bf16 I/O,
// fp16 MFMA operands, fp32 accumulation and state), gfx950.
//
// Same per-chunk algorithm and regrouping as chunk_fwd.hip ("Linear Attention, Visualized",
// section "Gated DeltaNet (GDN)", "Complete per-chunk algorithm"; column convention):
//
//   N = I + diag(beta) (K K^T (.) Gam)_strict,  T = N^{-1} diag(beta),  A = (Q K^T) (.) Gam
//   R = V - diag(e^G) K S^T,   Z = T R,   O = diag(e^G) Q S^T + A Z,
//   S^T <- e^{G_C} S^T + K^T diag(e^{G_C - G}) Z.
//
// The page notes that the chunk-local quantities (here N, T, A) can be formed for all chunks
// in parallel while the boundary pass threads the state through the chunks.  This kernel
// runs the two concurrently inside one workgroup of four waves:
//   * waves 0-1 (consumers) carry the state of 16 value channels each, run the whole
//     S-dependent chain of chunk i, and stage the inputs of later chunks into LDS;
//   * waves 2-3 (producers) form, for chunk i+1, A, the blocks of N below the diagonal and
//     the inverses of its four 16x16 diagonal blocks (forward substitution in fp32); the
//     consumer then applies N^{-1} diag(beta) by blocked forward substitution on MFMA.
// An iteration has two phases separated by workgroup barriers:
//   phase 0  consumers: chain of chunk i;         producers: Gram tiles and diagonal
//            G scan of chunk i+2 (wave 0)                    inverses of chunk i+1
//   phase 1  consumers: write o of chunk i; all waves: stage K, Q of chunk i+2 and V of i+1
// The global loads of chunk i+2 (and V of i+1) are issued in phase 0, interleaved with each
// wave's main MFMA loop.
// Every LDS buffer is written only in a phase where its previous contents are dead.
//
// MFMA 16x16x32 f16 conventions (l = lane, j = l & 15, g = l >> 4):
//   accumulator register r of lane l holds element (row 4g + r, column j);
//   an operand fragment of lane l is row/column j with the 8 reduction indices
//   {32kb + 4g + r} U {32kb + 16 + 4g + r}, r = 0..3.
// K and Q sit in LDS in natural channel order, so a fragment of 8 consecutive channels is
// ONE 16-byte read.  The state S^T is kept with its row index permuted within each 32-block
// (row 16h + 4gg + rr holds channel 8gg + 4h + rr, pperm below): then the accumulator of two
// vertically adjacent 16-row tiles of S^T IS the B fragment that pairs with those 8
// consecutive channels, and S^T, R and Z move between products in registers only.  K^T
// fragments (reduction over tokens) for the state update come from the token-major K copy
// through ds_read_b64_tr_b16, which hands lane i of each 16-lane group element (i & 3) of
// the 4-element rows addressed by lanes (i >> 2) + 4e, e = 0..3; reading channel columns
// pperm(16t + 4(i & 3)) gives S^T's permuted row order.
//
// Gated Delta Product ("Linear Attention, Visualized", sections "Gated Delta Product (GDP)"
// and "GDP as GDN over a virtual sequence"): the VIRT instantiation runs the same chain over
// the T n_h virtual steps m = n_h t + j of a GDP sequence (0-based t, j).  Keys, values and
// betas are stored per substep, so they already form the virtual sequence.  The query, the
// log-decay and the output are stored per real token: step m reads q_t only when
// j = n_h - 1 and g_t only when j = 0, and writes o only when j = n_h - 1.  On the other
// steps the buffer offset is set past the end of the real-token buffer, so the load returns
// zero (a zero query; log-decay 0, i.e. a = 1) and the store is dropped.
//
// The PREP instantiation fuses the step upstream of the chain: it takes raw projections and
// forms the rule's inputs on the fly, q = q_raw / ||q_raw||, k likewise (the pages' unit-norm
// convention), beta = sigmoid(beta_logit) and the Mamba-2 gate g = -e^{A_log[h]} softplus(dt +
// dt_bias[h]) ("Linear Attention, Visualized", "Optional: Constructing the decay gate").  The
// norms come from the staged 16-byte pieces (one K or Q row spans DK/8 consecutive lanes, so a
// DPP reduction inside each 16-lane row gives the row's sum of squares); each piece is scaled
// before its fp16 conversion.  The gate and beta are transformed where the scan reads them.
#include "chunk_common.h"

namespace gdr {

// Instantiations of the kernel: plain Gated DeltaNet, Gated Delta Product over virtual steps,
// Gated DeltaNet with fused input preparation.
constexpr int kPcPlain = 0, kPcGdp = 1, kPcPrep = 2;

struct PcArgs {
    int64_t T;         // steps per sequence (virtual steps T_real * nh for the VIRT kernel)
    int64_t Treal;     // tokens per sequence of q, g and o (= T unless VIRT)
    uint32_t nh;       // substeps per token (VIRT)
    uint32_t nh_magic; // ceil(2^32 / nh): m / nh = umulhi(m, nh_magic) for m < 2^23 (VIRT)
    int dv;
    int ntiles;  // d_v / 32
    int H;                  // heads (PREP: per-head gate parameters)
    const float* A_log;     // [H] (PREP)
    const float* dt_bias;   // [H] (PREP)
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* g;
    const float* beta;
    const float* S0;
    uint16_t* o;
    float* Sf;
};

template <int DK>
struct PcLds {
    static constexpr int C = kChunk;
    // halfs, rows of K / Q: a stride of 16 mod 128 halfs keeps both the 16-byte fragment
    // reads (row j, 8 channels at 8g) and the transposing reads (rows 4g + j/4) free of
    // LDS bank conflicts on gfx950
    static constexpr int LDK = DK + 16;
    static constexpr int LDC = C + 8;    // halfs, rows of C-wide fp16 matrices
    static constexpr int LDV = 80;       // bf16, rows (tokens) of the 32-channel V tile; a
                                         // transposing-read-friendly stride
    static constexpr int LDN = 16 + 4;   // floats, rows of a 16x16 fp32 block
    static constexpr int LDO = C + 8;    // bf16, rows of the output tile O^T
    // per-chunk factor table (floats):
    //   [0,64) G   [64,128) e^G   [128,192) e^{G_C - G}   [192,256) beta   [256] e^{G_C}
    //   [272,336)  cf[m]     = e^{Gend(blk(m)) - G_m}           (<= 1)
    //   [336,528)  rf[b][l]  = e^{G_l - Gend(b)}, b = 0..2        (<= 1 for blk(l) > b)
    //   [528,720)  rb[b][l]  = beta_l rf[b][l]
    // with Gend(b) = G at the last token of 16-token block b.
    static constexpr int SG = 0, SEG = 64, SEGR = 128, SB = 192, SEGC = 256, SCF = 272, SRF = 336, SRB = 528;
    static constexpr int NSM = 736;
    static constexpr int szK = C * LDK * 2;
    static constexpr int szC = C * LDC * 2;
    static constexpr int oKb0 = 0;
    static constexpr int oKb1 = oKb0 + szK;
    static constexpr int oQb0 = oKb1 + szK;
    static constexpr int oQb1 = oQb0 + szK;
    static constexpr int oAt0 = oQb1 + szK;   // A^T (column-major A), two chunks
    static constexpr int oAt1 = oAt0 + szC;
    static constexpr int oSm = oAt1 + szC;            // factor tables of three chunks
    static constexpr int LDX = 16 + 8;   // halfs, rows of a 16x16 fp16 block
    static constexpr int szX = 4 * 16 * LDX * 2;
    static constexpr int oVt = oSm + 3 * NSM * 4;
    static constexpr int oNt0 = oVt + C * LDV * 2;   // off-diagonal blocks of N^T (fp16), two chunks
    static constexpr int oNt1 = oNt0 + szC;
    static constexpr int oXd0 = oNt1 + szC;          // X_bb^T, the diagonal blocks of N^{-1} (fp16), two chunks
    static constexpr int oXd1 = oXd0 + szX;
    static constexpr int oNd = oXd1 + szX;           // diagonal blocks of N^T (fp32)
    static constexpr int oOt = oNd + 4 * 16 * LDN * 4;  // O^T of the consumer chunk (bf16)
    static constexpr int total = oOt + 32 * LDO * 2;
    static_assert(total <= 160 * 1024, "LDS budget of one gfx950 CU exceeded");
    static_assert((oAt0 | oAt1 | oSm | oVt | oNt0 | oNt1 | oXd0 | oXd1 | oNd | oOt) % 16 == 0, "alignment");
};

template <int DK, int MODE>
__global__ __launch_bounds__(256, 1) void chunk_fwd_pc_kernel(const PcArgs a) {
    constexpr bool VIRT = MODE == kPcGdp, PREP = MODE == kPcPrep;
    using L = PcLds<DK>;
    constexpr int C = kChunk;
    constexpr int NKB = DK / 32;      // 32-deep reduction blocks over d_k
    constexpr int NST = DK / 16;      // 16-row tiles of S^T
    constexpr int KVL = C * DK / 8 / 256;  // 16-byte vectors of one K chunk per lane
    extern __shared__ __attribute__((aligned(16))) char smem[];
    auto Kb = [&](int b) { return reinterpret_cast<_Float16*>(smem + (b ? L::oKb1 : L::oKb0)); };
    auto Qb = [&](int b) { return reinterpret_cast<_Float16*>(smem + (b ? L::oQb1 : L::oQb0)); };
    auto At = [&](int b) { return reinterpret_cast<_Float16*>(smem + (b ? L::oAt1 : L::oAt0)); };
    // factor table of chunk c: buffer c mod 3, so the scan of chunk c+2 never meets the
    // tables that the consumer (chunk c) and the producers (chunk c+1) are reading
    // (the buffer index is passed in, kept by rotation: no 64-bit division in the loop)
    auto Sm = [&](int m3) { return reinterpret_cast<float*>(smem + L::oSm + m3 * L::NSM * 4); };
    uint16_t* Vt = reinterpret_cast<uint16_t*>(smem + L::oVt);  // V tile, bf16 [token][channel]
    auto Ntb = [&](int b) { return reinterpret_cast<_Float16*>(smem + (b ? L::oNt1 : L::oNt0)); };
    auto Xdb = [&](int b) { return reinterpret_cast<_Float16*>(smem + (b ? L::oXd1 : L::oXd0)); };
    float* Nd = reinterpret_cast<float*>(smem + L::oNd);
    _Float16* Ot = reinterpret_cast<_Float16*>(smem + L::oOt);  // holds bf16 bit patterns

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, j = l & 15, g = l >> 4;
    const bool consumer = w < 2;
    const int p = w - 2;           // producer index (valid when !consumer)
    // the producers' work per chunk is the longer of the two roles: let them win arbitration
    // for the CU's shared LDS and memory pipelines
    if (!consumer) __builtin_amdgcn_s_setprio(2);
    const int vi = xcd_major_index(blockIdx.x, gridDim.x);
    const int64_t bh = vi / a.ntiles;
    const int dv0 = (vi % a.ntiles) * 32;
    const int64_t T = a.T;
    const int DV = a.dv;
    const int64_t Tr = VIRT ? a.Treal : T;  // rows of q, g and o per sequence
    const uint32_t qbytes = (uint32_t)(Tr * DK * 2), gbytes = (uint32_t)(Tr * 4), obytes = (uint32_t)(Tr * DV * 2);
    const auto rq = make_rsrc(a.q + bh * Tr * DK, qbytes);
    const auto rk = make_rsrc(a.k + bh * T * DK, (uint32_t)(T * DK * 2));
    const auto rv = make_rsrc(a.v + bh * T * DV, (uint32_t)(T * DV * 2));
    const auto rg = make_rsrc(a.g + bh * Tr, gbytes);
    const auto rb = make_rsrc(a.beta + bh * T, (uint32_t)(T * 4));
    const auto ro = make_rsrc(a.o + bh * Tr * DV, obytes);
    // virtual step m -> (real token, substep) of a Gated Delta Product sequence
    auto vtok = [&](uint32_t m) { return __umulhi(m, a.nh_magic); };
    // gate parameters of this head (PREP): lambda = e^{A_log}, the bias of dt
    float lam = 0.0f, dtb = 0.0f;
    if constexpr (PREP) {
        const int h = (int)(bh % a.H);
        lam = fast_exp(a.A_log[h]);
        dtb = a.dt_bias[h];
    }
    const int dvc = dv0 + 16 * w;  // consumer's first value channel
    const int64_t nC = (T + C - 1) / C;

    // 16-deep product: lane (j, g) gives A[j][4g..4g+3] and B[4g..4g+3][j]
    auto mma16k16 = [](float4v& acc, const half4& a4, const half4& b4) {
        acc = __builtin_amdgcn_mfma_f32_16x16x16f16(a4, b4, acc, 0, 0, 0);
    };
    // operand fragment (rows 16*rt.., 8 reduction indices of block kb) of a row-major matrix
    // whose reduction index runs along a column-major copy: transposing reads of the
    // column-major matrix M^T at rows 32kb + 4g + (j >> 2) (+16) and columns col0 + 4(j & 3).
    auto trfrag = [&](const _Float16* base, int ld, int kb, int col) {
        const _Float16* p0 = base + (32 * kb + 4 * g + (j >> 2)) * ld + col;
        return cat8(ldtr(p0), ldtr(p0 + 16 * ld));
    };

    // ---- zero the operand scratch whose never-written parts are read as structural zeros
    for (int i = tid; i < (L::total - L::oAt0) / 16; i += 256)
        reinterpret_cast<uint4*>(smem + L::oAt0)[i] = uint4{0u, 0u, 0u, 0u};

    // ---- registers carried across phases.  A wave plays one role for the whole kernel, so
    // the two roles share one array: consumers keep the state S^T (fp32 accumulators) and
    // its fp16 operand copy; producers keep blocks of N^{-1}.
    //   consumer: [0, 4*NST) S^T tiles   [4*NST, 4*NST + 4*NKB) fp16 copy of S^T
    //   every wave: [oKR, NCARRY) its share of the prefetched K, Q, V, g, beta
    constexpr int oSB = 4 * NST;
    constexpr int oKR = oSB + 4 * NKB;
    constexpr int oQR = oKR + 4 * KVL, oVR = oQR + 4 * KVL, oGR = oVR + 4;
    constexpr int NCARRY = oGR + 2;
    uint32_t cr[NCARRY];
#pragma unroll
    for (int i = 0; i < NCARRY; ++i) cr[i] = 0u;
    auto getf4 = [&](int o) { return float4v{__uint_as_float(cr[o]), __uint_as_float(cr[o + 1]), __uint_as_float(cr[o + 2]), __uint_as_float(cr[o + 3])}; };
    auto setf4 = [&](int o, const float4v& v) {
#pragma unroll
        for (int e = 0; e < 4; ++e) cr[o + e] = __float_as_uint(v[e]);
    };
    auto geth8 = [&](int o) { return __builtin_bit_cast(half8, uint4{cr[o], cr[o + 1], cr[o + 2], cr[o + 3]}); };
    auto seth8 = [&](int o, const half8& h) {
        const uint4 u = __builtin_bit_cast(uint4, h);
        cr[o] = u.x; cr[o + 1] = u.y; cr[o + 2] = u.z; cr[o + 3] = u.w;
    };
    auto getu4 = [&](int o) { return uint4{cr[o], cr[o + 1], cr[o + 2], cr[o + 3]}; };
    auto setu4 = [&](int o, const uint4& u) { cr[o] = u.x; cr[o + 1] = u.y; cr[o + 2] = u.z; cr[o + 3] = u.w; };

    if (consumer) {
        if (a.S0 != nullptr) {
            const float* s0 = a.S0 + bh * (int64_t)DV * DK + (int64_t)(dvc + j) * DK;
#pragma unroll
            for (int t = 0; t < NST; ++t) setf4(4 * t, ld4f(s0 + pperm(16 * t + 4 * g)));
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) seth8(oSB + 4 * kb, pack8(getf4(8 * kb), getf4(8 * kb + 4)));
    }

    // ---- staging (all 256 lanes): global -> registers -> LDS.  Past the sequence end the
    // buffer loads return zeros, i.e. identity tokens.
    const int pt = tid;
    // Global loads of one iteration, in KVL parts: part u brings the lane's u-th 16-byte
    // pieces of K and Q of chunk cs; part 0 also V of chunk cv and (wave 0) g, beta of cs.
    // The parts are issued between the MFMAs of each wave's main product loop, so the
    // vector-memory queue drains while the matrix pipe is busy.
    auto issue_part = [&](int u, int64_t cs_, int64_t cv_) {
        const uint32_t t0 = (uint32_t)(cs_ * C);
        const int idx = pt + 256 * u, row = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
        const uint32_t off = ((t0 + row) * DK + col) * 2;
        uint32_t offq = off;
        if constexpr (VIRT) {  // q_t on the last substep of token t, zero elsewhere
            const uint32_t m = t0 + row, tr = vtok(m);
            offq = m - tr * a.nh == a.nh - 1 ? (tr * DK + col) * 2 : qbytes;
        }
        setu4(oKR + 4 * u, bld16(rk, off));
        setu4(oQR + 4 * u, bld16(rq, offq));
        if (u == 0) {
            const uint32_t tv = (uint32_t)(cv_ * C);
            setu4(oVR, bld16(rv, ((tv + (pt >> 2)) * DV + dv0 + (pt & 3) * 8) * 2));
            if (w == 0) {
                uint32_t offg = (t0 + l) * 4;
                if constexpr (VIRT) {  // log-decay g_t on the first substep, 0 elsewhere
                    const uint32_t m = t0 + l, tr = vtok(m);
                    offg = m - tr * a.nh == 0 ? tr * 4 : gbytes;
                }
                cr[oGR] = __float_as_uint(bld4(rg, offg));
                cr[oGR + 1] = __float_as_uint(bld4(rb, (t0 + l) * 4));
            }
        }
    };
    auto issue_all = [&](int64_t cs_, int64_t cv_) {
#pragma unroll
        for (int u = 0; u < KVL; ++u) issue_part(u, cs_, cv_);
    };
    // PREP: a row piece of 8 bf16 values divided by its row's L2 norm, in fp16.  The row's
    // DK/8 pieces sit in consecutive lanes of one 16-lane DPP row; quad_perm xor 1, xor 2,
    // row_half_mirror (and row_mirror for 16 lanes) leave the row sum in every lane.
    auto unit_half8 = [&](const uint4& u) {
        const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
        float x[8], ss = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = __uint_as_float(wv[e] << 16);
            x[2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
        ss += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0xB1, 0xf, 0xf, false));
        ss += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0x4E, 0xf, 0xf, false));
        ss += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0x141, 0xf, 0xf, false));
        if constexpr (DK == 128)
            ss += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0x140, 0xf, 0xf, false));
        const float inv = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-12f));  // 1 / max(||x||, 1e-6)
        half8 h;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (_Float16)(x[e] * inv);
        return h;
    };
    auto stage_kq = [&](int64_t c) {
        const int buf = (int)(c & 1);
#pragma unroll
        for (int u = 0; u < KVL; ++u) {
            const int idx = pt + 256 * u, row = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            if constexpr (PREP) {
                *reinterpret_cast<half8*>(Kb(buf) + row * L::LDK + col) = unit_half8(getu4(oKR + 4 * u));
                *reinterpret_cast<half8*>(Qb(buf) + row * L::LDK + col) = unit_half8(getu4(oQR + 4 * u));
            } else {
                *reinterpret_cast<half8*>(Kb(buf) + row * L::LDK + col) = bf16x8_to_half8(getu4(oKR + 4 * u));
                *reinterpret_cast<half8*>(Qb(buf) + row * L::LDK + col) = bf16x8_to_half8(getu4(oQR + 4 * u));
            }
        }
    };
    // In-chunk cumulative log-decay G and the per-chunk factor table of chunk c (wave 0,
    // from the g and beta values its issue_part(0, c, ..) loaded).
    // PREP: past the sequence end the raw loads are zeros, which the transforms would turn
    // into g = -lambda softplus(b) and beta = 1/2; such tokens are set back to identity tokens.
    auto scan = [&](int m3, int64_t chunk) {
        float gl = __uint_as_float(cr[oGR]);
        const bool live = !PREP || chunk * C + l < T;
        if constexpr (PREP) {  // g = -lambda softplus(dt + b), softplus(z) = max(z, 0) + log(1 + e^{-|z|})
            const float z = gl + dtb;
            gl = live ? -lam * (fmaxf(z, 0.0f) + __logf(1.0f + fast_exp(-fabsf(z)))) : 0.0f;
        }
        const float x = wave_inclusive_scan(gl);
        const float GC = lane_value(x, 63);
        float ge[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) ge[b] = lane_value(x, 16 * b + 15);
        const int blk = l >> 4;
        float beta = __uint_as_float(cr[oGR + 1]);
        if constexpr (PREP) beta = live ? 1.0f / (1.0f + fast_exp(-beta)) : 0.0f;
        float* sm = Sm(m3);
        sm[L::SG + l] = x;
        sm[L::SEG + l] = fast_exp(x);
        sm[L::SEGR + l] = fast_exp(GC - x);
        sm[L::SB + l] = beta;
        if (l == 0) sm[L::SEGC] = fast_exp(GC);
        sm[L::SCF + l] = fast_exp(ge[blk] - x);
#pragma unroll
        for (int b = 0; b < 3; ++b) {
            const float f = blk > b ? fast_exp(x - ge[b]) : 0.0f;
            sm[L::SRF + 64 * b + l] = f;
            sm[L::SRB + 64 * b + l] = beta * f;
        }
    };
    auto stage_v = [&]() {  // V tile as loaded: bf16 [token][32 channels]
        *reinterpret_cast<uint4*>(Vt + (pt >> 2) * L::LDV + (pt & 3) * 8) = getu4(oVR);
    };

    lds_barrier();  // zero-fill done
    if (nC > 0) {
        issue_all(0, 0);
        stage_kq(0);
        if (w == 0) scan(0, 0);  // chunk 0 -> buffer 0
    }
    lds_barrier();

    // Gram tiles of one producer wave.  Wave 2 forms KK {00,10,11,20,21,30,31} and
    // QK {00,10,11}; wave 3 forms KK {22,32,33} and QK {20,21,22,30,31,32,33}.  Per
    // reduction block each wave loads its 6 distinct row fragments once (K row tiles 0-3, Q
    // row tiles 2P, 2P+1) one block ahead, then issues 10 independent MFMAs.  The epilogue
    // applies the decay (factorised through the per-chunk table off the diagonal, exact on
    // it) and beta, and stores each tile column-major: a lane's 4 accumulator rows are
    // contiguous there.
    auto gram_wave = [&](const _Float16* Kp, const _Float16* Qp, const float* sm, _Float16* Ap, _Float16* Np,
                         const int P, int64_t cs_, int64_t cv_) {
        constexpr int NT = 10;
        const int tq[2][NT] = {{0, 0, 0, 0, 0, 0, 0, 1, 1, 1}, {0, 0, 0, 1, 1, 1, 1, 1, 1, 1}};
        const int ti_[2][NT] = {{0, 1, 1, 2, 2, 3, 3, 0, 1, 1}, {2, 3, 3, 2, 2, 2, 3, 3, 3, 3}};
        const int tj_[2][NT] = {{0, 0, 1, 0, 1, 0, 1, 0, 0, 1}, {2, 2, 3, 0, 1, 2, 0, 1, 2, 3}};
        auto load6 = [&](half8* f, int kb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) f[r] = ld8(Kp + (16 * r + j) * L::LDK + 32 * kb + 8 * g);
#pragma unroll
            for (int r = 0; r < 2; ++r) f[4 + r] = ld8(Qp + (16 * (2 * P + r) + j) * L::LDK + 32 * kb + 8 * g);
        };
        // Per-tile scale factors, formed between the products so that their LDS reads and
        // exponentials overlap the MFMAs: element (l0 + r, m) of tile t is acc * fr[t][r] * fc[t]
        // off the diagonal; on it fr already holds the exact decay (and beta for N) with the
        // causal mask applied.
        float4v fr[NT];
        float fc[NT];
        auto factors = [&](const int t) {
            const int ti = ti_[P][t], tj = tj_[P][t];
            const bool isQ = tq[P][t];
            const int m = 16 * tj + j, l0 = 16 * ti + 4 * g;
            if (ti != tj) {
                fr[t] = ld4f(sm + (isQ ? L::SRF : L::SRB) + 64 * tj + l0);
                fc[t] = sm[L::SCF + m];
            } else {
                const float Gm = sm[L::SG + m];
                const float4v Gl = ld4f(sm + L::SG + l0);
                const float4v bl = isQ ? float4v{1.0f, 1.0f, 1.0f, 1.0f} : ld4f(sm + L::SB + l0);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool keep = isQ ? (m <= l0 + r) : (m < l0 + r);
                    fr[t][r] = keep ? bl[r] * fast_exp(Gl[r] - Gm) : 0.0f;
                }
                fc[t] = 1.0f;
            }
        };
        float4v acc[NT];
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
                if (t == 1) issue_part(kb, cs_, cv_);
            }
            // the epilogue's factors, computed while the matrix pipe works through this block
            if (kb < 2) {
#pragma unroll
                for (int t = 5 * kb; t < 5 * kb + 5; ++t) factors(t);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int ti = ti_[P][t], tj = tj_[P][t];
            const bool isQ = tq[P][t];
            const int m = 16 * tj + j;            // this lane's column
            const int l0 = 16 * ti + 4 * g;       // first of its 4 rows
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[t][r] * fr[t][r] * fc[t];
            if (ti == tj && !isQ) {
                // N^T diagonal block ti, column j: rows 4g..4g+3, unit diagonal
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (m == l0 + r) v[r] = 1.0f;
                *reinterpret_cast<float4v*>(Nd + (ti * 16 + j) * L::LDN + 4 * g) = float4v{v[0], v[1], v[2], v[3]};
            } else {
                _Float16* dst = (isQ ? Ap : Np) + m * L::LDC + l0;
                *reinterpret_cast<half4*>(dst) = half4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
            }
        }
    };

    // factor-table buffers (chunk mod 3) of the consumer, producer and scanned chunks
    int mc = 2, mp = 0, ms = 1;
    for (int64_t it = -1; it < nC; ++it, mc = mp, mp = ms, ms = (ms == 2 ? 0 : ms + 1)) {
        const int64_t cc = it;        // consumer chunk
        const int64_t cp = it + 1;    // producer chunk (N blocks, diagonal inverses, A)
        const int64_t cs = it + 2;    // chunk whose K, Q are staged in phase 1
        const int bc = (int)(cc & 1), bp = (int)(cp & 1);

        // ======================= phase 0 =======================
        // Loads are unconditional: past the sequence end the buffer loads return zeros, and
        // staging those zeros touches only buffers no later chunk reads.
        if (consumer) {
            if (cc < 0) issue_all(cs, cp);
            if (cc >= 0) {
                const _Float16* Kc = Kb(bc);
                const _Float16* Qc = Qb(bc);
                const _Float16* Ac = At(bc);
                const _Float16* Nc = Ntb(bc);
                const _Float16* Xc = Xdb(bc);
                const float* sm = Sm(mc);
                // The LDS operand fragments of each group of MFMAs are issued one group ahead
                // (double-buffered registers), and sched_barrier pins that order: left alone,
                // the scheduler serialises every ds_read with the MFMA that consumes it.
                auto kfrag = [&](int ti, int kb) { return ld8(Kc + (16 * ti + j) * L::LDK + 32 * kb + 8 * g); };
                auto qfrag = [&](int ti, int kb) { return ld8(Qc + (16 * ti + j) * L::LDK + 32 * kb + 8 * g); };
                // P_K = K S^T, P_Q = Q S^T  (rows = tokens), reduction over d_k in NKB blocks
                float4v PK[4], PQ[4];
                half8 fa[8], fb[8];
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
                    PK[ti] = zero4();
                    PQ[ti] = zero4();
                    fa[ti] = kfrag(ti, 0);
                    fa[4 + ti] = qfrag(ti, 0);
                }
                float4v eg[4], vv[4], bt[4];
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
                    eg[ti] = ld4f(sm + L::SEG + 16 * ti + 4 * g);
                    // V[16ti + 4g + r][16w + j] through a transposing read, widened from bf16
                    const uint2 vb = __builtin_bit_cast(
                        uint2, ldtr(reinterpret_cast<const _Float16*>(Vt) + (16 * ti + 4 * g + (j >> 2)) * L::LDV +
                                    16 * w + 4 * (j & 3)));
                    vv[ti] = float4v{__uint_as_float(vb.x << 16), __uint_as_float(vb.x & 0xffff0000u),
                                     __uint_as_float(vb.y << 16), __uint_as_float(vb.y & 0xffff0000u)};
                    bt[ti] = ld4f(sm + L::SB + 16 * ti + 4 * g);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    half8* cur = (kb & 1) ? fb : fa;
                    half8* nxt = (kb & 1) ? fa : fb;
                    if (kb + 1 < NKB) {
#pragma unroll
                        for (int ti = 0; ti < 4; ++ti) {
                            nxt[ti] = kfrag(ti, kb + 1);
                            nxt[4 + ti] = qfrag(ti, kb + 1);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    const half8 sb = geth8(oSB + 4 * kb);
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti) {
                        mma16(PK[ti], cur[ti], sb);
                        mma16(PQ[ti], cur[4 + ti], sb);
                        if (ti == 0) issue_part(kb, cs, cp);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                // operands of the block substitution: X_bb (diagonal inverses) and the N blocks
                // below the diagonal, as A fragments from their column-major copies; rows of A
                half4 xf[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) xf[b] = ldtr(Xc + (16 * b + 4 * g + (j >> 2)) * L::LDX + 4 * (j & 3));
                const half4 n10 = ldtr(Nc + (4 * g + (j >> 2)) * L::LDC + 16 + 4 * (j & 3));
                const half8 n2x = trfrag(Nc, L::LDC, 0, 32 + 4 * (j & 3));   // [N20 N21]
                const half8 n3x = trfrag(Nc, L::LDC, 0, 48 + 4 * (j & 3));   // [N30 N31]
                const half4 n32 = ldtr(Nc + (32 + 4 * g + (j >> 2)) * L::LDC + 48 + 4 * (j & 3));
                half8 af[6];
#pragma unroll
                for (int ti = 0, n = 0; ti < 4; ++ti) {
#pragma unroll
                    for (int kb = 0; kb <= (ti >> 1); ++kb, ++n) af[n] = trfrag(Ac, L::LDC, kb, 16 * ti + 4 * (j & 3));
                }
                float4v er[4];
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) er[ti] = ld4f(sm + L::SEGR + 16 * ti + 4 * g);
                const float eGC = sm[L::SEGC];
                __builtin_amdgcn_sched_barrier(0);
                // R' = diag(beta) (V - e^G P_K) ;  O_hist = e^G P_Q
                float4v Rb[4], Oh[4];
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        Rb[ti][r] = bt[ti][r] * (vv[ti][r] - eg[ti][r] * PK[ti][r]);
                        Oh[ti][r] = eg[ti][r] * PQ[ti][r];
                    }
                }
                // Z = N^{-1} R' by blocked forward substitution over the 16-token blocks:
                //   Z_b = X_bb (R'_b - sum_{b' < b} N_{b b'} Z_{b'})
                auto h4 = [](const float4v& x) { return half4{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]}; };
                auto sub4 = [](float4v a4, const float4v& b4) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) a4[r] -= b4[r];
                    return a4;
                };
                float4v Zz[4], y;
                Zz[0] = zero4();
                mma16k16(Zz[0], xf[0], h4(Rb[0]));
                y = zero4();
                mma16k16(y, n10, h4(Zz[0]));
                Zz[1] = zero4();
                mma16k16(Zz[1], xf[1], h4(sub4(Rb[1], y)));
                const half8 z01 = pack8(Zz[0], Zz[1]);
                y = zero4();
                mma16(y, n2x, z01);
                Zz[2] = zero4();
                mma16k16(Zz[2], xf[2], h4(sub4(Rb[2], y)));
                y = zero4();
                mma16(y, n3x, z01);
                mma16k16(y, n32, h4(Zz[2]));
                Zz[3] = zero4();
                mma16k16(Zz[3], xf[3], h4(sub4(Rb[3], y)));
                // A operand of the state update: K^T[16t + i][tokens] from the token-major K
                // copy (d_k permuted).  First half of the tiles now.
                auto ktfrag = [&](int t, int kb) { return trfrag(Kc, L::LDK, kb, pperm(16 * t + 4 * (j & 3))); };
                half8 kt0[NST], kt1[NST];
#pragma unroll
                for (int t = 0; t < NST / 2; ++t) {
                    kt0[t] = ktfrag(t, 0);
                    kt1[t] = ktfrag(t, 1);
                }
                __builtin_amdgcn_sched_barrier(0);
                // O = O_hist + A Z, rounded to bf16 into this wave's rows of O^T (written to
                // o in phase 1).
                const half8 zB[2] = {z01, pack8(Zz[2], Zz[3])};
#pragma unroll
                for (int ti = 0, n = 0; ti < 4; ++ti) {
                    float4v acc = Oh[ti];
#pragma unroll
                    for (int kb = 0; kb <= (ti >> 1); ++kb, ++n) mma16(acc, af[n], zB[kb]);
                    *reinterpret_cast<uint2*>(Ot + (16 * w + j) * L::LDO + 16 * ti + 4 * g) =
                        uint2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
                }
                // S^T <- e^{G_C} S^T + K^T diag(e^{G_C - G}) Z
                float4v zs[4];
#pragma unroll
                for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                    for (int r = 0; r < 4; ++r) zs[ti][r] = er[ti][r] * Zz[ti][r];
                const half8 sZ0 = pack8(zs[0], zs[1]), sZ1 = pack8(zs[2], zs[3]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int t = NST / 2; t < NST; ++t) {
                    kt0[t] = ktfrag(t, 0);
                    kt1[t] = ktfrag(t, 1);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int t = 0; t < NST; ++t) {
                    float4v st = getf4(4 * t);
#pragma unroll
                    for (int r = 0; r < 4; ++r) st[r] *= eGC;
                    mma16(st, kt0[t], sZ0);
                    mma16(st, kt1[t], sZ1);
                    setf4(4 * t, st);
                }
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) seth8(oSB + 4 * kb, pack8(getf4(8 * kb), getf4(8 * kb + 4)));
            }
            if (w == 0) scan(ms, cs);
        } else {
          if (cp >= nC) issue_all(cs, cp);
          if (cp < nC) {
            const _Float16* Kp = Kb(bp);
            const _Float16* Qp = Qb(bp);
            if (p == 0) gram_wave(Kp, Qp, Sm(mp), At(bp), Ntb(bp), 0, cs, cp);
            else gram_wave(Kp, Qp, Sm(mp), At(bp), Ntb(bp), 1, cs, cp);
            lds_fence();
            // diagonal 16x16 blocks 2p, 2p+1 of X = N^{-1}, column-oriented forward
            // substitution: lane (block, jc) builds column jc; after x[i] is final it is
            // eliminated from the later rows, x[t] -= N[t][i] x[i] for t > i (column i of N
            // is row i of the stored N^T block).  Stored as X_bb^T (row jc = column jc of X_bb).
            {
                const int b = 2 * p + ((l >> 4) & 1), jc = j;
                const float* nb = Nd + b * 16 * L::LDN;
                // all rows first: the substitution is a chain of dependent FMAs, and waiting
                // for each row's LDS read inside it would serialise the latencies
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
                    _Float16* xr = Xdb(bp) + (16 * b + jc) * L::LDX;
                    *reinterpret_cast<half8*>(xr) = h0;
                    *reinterpret_cast<half8*>(xr + 8) = h1;
                }
            }
          }
        }
        lds_barrier();

        // ======================= phase 1 =======================
        // o of chunk cc: each consumer wave reads its rows of O^T back transposed (a lane gets
        // 8 consecutive channels of one token) and writes them with 16-byte stores.
        if (consumer && cc >= 0) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int tb = 32 * s2 + 16 * (g >> 1), d = 16 * w + 8 * (g & 1);
                const _Float16* rp = Ot + (d + (j >> 2)) * L::LDO + tb + 4 * (j & 3);
                const uint2 lo = __builtin_bit_cast(uint2, ldtr(rp));
                const uint2 hi = __builtin_bit_cast(uint2, ldtr(rp + 4 * L::LDO));
                uint32_t offo = ((uint32_t)(cc * C + tb + j) * DV + dv0 + d) * 2;
                if constexpr (VIRT) {  // only the last substep of a token has an output
                    const uint32_t m = (uint32_t)(cc * C + tb + j), tr = vtok(m);
                    offo = m - tr * a.nh == a.nh - 1 ? (tr * DV + dv0 + d) * 2 : obytes;
                }
                bst16(ro, offo, uint4{lo.x, lo.y, hi.x, hi.y});
            }
        }
        // The consumer is done with K, Q of chunk cc (= cs mod 2) and with V of cc.
        stage_kq(cs);
        stage_v();
        lds_barrier();
    }

    if (consumer && a.Sf != nullptr) {
        float* sf = a.Sf + bh * (int64_t)DV * DK + (int64_t)(dvc + j) * DK;
#pragma unroll
        for (int t = 0; t < NST; ++t) *reinterpret_cast<float4v*>(sf + pperm(16 * t + 4 * g)) = getf4(4 * t);
    }
}

template <int DK, int MODE>
static hipError_t launch_pc(const PcArgs& a, int64_t nwg, hipStream_t st) {
    using L = PcLds<DK>;
    auto kern = chunk_fwd_pc_kernel<DK, MODE>;
    static std::atomic<uint64_t> lds_enabled{0};  // one bit per device
    if (const hipError_t e = enable_dynamic_lds(kern, L::total, lds_enabled); e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(256), L::total, st, a);
    return hipGetLastError();
}

// T counts real tokens; nh > 1 runs a Gated Delta Product over the T * nh virtual steps
// (k, v, beta hold T * nh rows per sequence; q, g, o hold T).
hipError_t chunk_fwd_pc_dispatch(int64_t BH, int64_t T, int nh, int dk, int dv, const void* q, const void* k,
                                 const void* v, const float* g, const float* beta, const float* S0, void* o,
                                 float* Sf, hipStream_t st) {
    PcArgs a;
    a.T = T * nh;
    a.Treal = T;
    a.nh = (uint32_t)nh;
    a.nh_magic = nh > 1 ? (uint32_t)(((uint64_t(1) << 32) + nh - 1) / nh) : 0u;
    a.H = 1;
    a.A_log = nullptr;
    a.dt_bias = nullptr;
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
    if (nh > 1) {
        if (dk == 128) return launch_pc<128, kPcGdp>(a, nwg, st);
        return launch_pc<64, kPcGdp>(a, nwg, st);
    }
    if (dk == 128) return launch_pc<128, kPcPlain>(a, nwg, st);
    return launch_pc<64, kPcPlain>(a, nwg, st);
}

// Gated DeltaNet from raw projections: q_raw, k_raw [BH][T][dk] bf16 (normalised here),
// dt and beta_logit [BH][T], A_log and dt_bias [H] (bh mod H is the head).
hipError_t chunk_fwd_pc_prep_dispatch(int64_t BH, int64_t H, int64_t T, int dk, int dv, const void* q_raw,
                                      const void* k_raw, const void* v, const float* dt, const float* A_log,
                                      const float* dt_bias, const float* beta_logit, const float* S0, void* o,
                                      float* Sf, hipStream_t st) {
    PcArgs a;
    a.T = T;
    a.Treal = T;
    a.nh = 1;
    a.nh_magic = 0u;
    a.dv = dv;
    a.ntiles = dv / 32;
    a.H = (int)H;
    a.A_log = A_log;
    a.dt_bias = dt_bias;
    a.q = static_cast<const uint16_t*>(q_raw);
    a.k = static_cast<const uint16_t*>(k_raw);
    a.v = static_cast<const uint16_t*>(v);
    a.g = dt;
    a.beta = beta_logit;
    a.S0 = S0;
    a.o = static_cast<uint16_t*>(o);
    a.Sf = Sf;
    const int64_t nwg = BH * a.ntiles;
    if (dk == 128) return launch_pc<128, kPcPrep>(a, nwg, st);
    return launch_pc<64, kPcPrep>(a, nwg, st);
}

}  // namespace gdr
