// gdr_api.hip -- host side of the libgdr C ABI: argument validation and kernel dispatch.
// Declarations and the contract of every entry point are in include/gdr.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdr.h"

namespace gdr {
hipError_t chunk_fwd_dispatch(int64_t BH, int64_t T, int dk, int dv, bool bf16, bool channel, const void* q,
                              const void* k, const void* v, const float* g, const float* beta, const float* S0,
                              void* o, float* Sf, hipStream_t st);
hipError_t chunk_fwd_pc_dispatch(int64_t BH, int64_t T, int nh, int dk, int dv, const void* q, const void* k,
                                 const void* v, const float* g, const float* beta, const float* S0, void* o,
                                 float* Sf, hipStream_t st);
hipError_t chunk_kda_dispatch(int64_t BH, int64_t T, int dk, int dv, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, const float* S0, void* o, float* Sf, hipStream_t st);
hipError_t chunk_split_dispatch(int64_t BH, int64_t T, int nh, int dk, int dv, const void* q, const void* k,
                                const void* v, const float* g, const float* beta, const float* S0, void* o, float* Sf,
                                void* ws, hipStream_t st);
int64_t chunk_split_workspace_bytes(int64_t BH, int64_t T);
int64_t chunk_split_prep_workspace_bytes(int64_t BH, int64_t T, int dk);
hipError_t chunk_split_prep_dispatch(int64_t BH, int64_t H, int64_t T, int dk, int dv, const void* q_raw,
                                     const void* k_raw, const void* v, const float* dt, const float* A_log,
                                     const float* dt_bias, const float* beta_logit, const float* S0, void* o,
                                     float* Sf, void* ws, hipStream_t st);
hipError_t chunk_kda_ut_dispatch(int64_t BH, int64_t T, int dk, const void* q, const void* k, const float* g,
                                 const float* beta, const float* eg, void* ws, hipStream_t st);
int64_t chunk_kda_ws_halfs(int dk);
hipError_t chunk_state_kda_dispatch(int64_t BH, int64_t T, int dk, int dv, const void* v, const float* wg,
                                    const float* S0, void* o, float* Sf, const void* ws, hipStream_t st);
hipError_t chunk_fwd_pc_prep_dispatch(int64_t BH, int64_t H, int64_t T, int dk, int dv, const void* q_raw,
                                      const void* k_raw, const void* v, const float* dt, const float* A_log,
                                      const float* dt_bias, const float* beta_logit, const float* S0, void* o,
                                      float* Sf, hipStream_t st);
hipError_t frame_dispatch(int64_t BH, int64_t T, int n, int dk, int dv, bool channel, const void* q, const void* k,
                          const void* v, const float* gamma, const float* g, const float* S0, void* o, float* Sf,
                          void* ws, hipStream_t st);
int64_t frame_workspace_bytes(int64_t BH, int64_t T, int n, int dk, int dv);
hipError_t chunk_gdn2_dispatch(int64_t BH, int64_t T, int dk, int dv, const void* q, const void* k, const void* v,
                               const float* g, const float* b, const float* w, const float* S0, void* o, float* Sf,
                               hipStream_t st);
hipError_t decode_dispatch(int64_t NH, int dk, int dv, bool bf16, bool channel, const void* q, const void* k,
                           const void* v, const float* g, const float* beta, float* S, void* o, hipStream_t st);
}  // namespace gdr

namespace {

constexpr int kVersion = 10000 * 0 + 100 * 1 + 0;
constexpr int64_t kMaxGrid = 0x7fffffff;
// The kernels address one sequence with 32-bit byte offsets: T * d * 4 stays below 2^32.
constexpr int64_t kMaxT = int64_t(1) << 22;
// Chunk length of the chunked kernels.
constexpr int64_t kChunkLen = 64;
// Substeps per token of the Gated Delta Product forward.
constexpr int kMaxNh = 16;

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

// Byte ranges [p, p + n) and [q, q + m) overlap.
bool overlaps(const void* p, int64_t n, const void* q, int64_t m) {
    if (!p || !q || n <= 0 || m <= 0) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + static_cast<uintptr_t>(m) && b < a + static_cast<uintptr_t>(n);
}

gdr_status check_common(int d_k, int d_v, int io_dtype, int gate) {
    if (io_dtype != GDR_BF16 && io_dtype != GDR_F32) return GDR_ERR_DTYPE;
    if (gate != GDR_GATE_SCALAR && gate != GDR_GATE_CHANNEL) return GDR_ERR_INVALID_ARG;
    if (d_k != 64 && d_k != 128) return GDR_ERR_SHAPE;
    if (d_v < 32 || d_v > 256 || (d_v % 32) != 0) return GDR_ERR_SHAPE;
    return GDR_OK;
}

}  // namespace

extern "C" {

int gdr_version(void) { return kVersion; }

const char* gdr_status_string(int status) {
    switch (status) {
        case GDR_OK: return "success";
        case GDR_ERR_INVALID_ARG: return "invalid argument (null buffer, negative size or bad enum)";
        case GDR_ERR_SHAPE: return "unsupported size (d_k must be 64 or 128, d_v a multiple of 32 in [32, 256])";
        case GDR_ERR_DTYPE: return "unsupported io dtype (GDR_BF16 or GDR_F32)";
        case GDR_ERR_UNSUPPORTED: return "valid but unsupported combination of arguments";
        case GDR_ERR_HIP: return "HIP runtime error while enqueuing the kernel";
        default: return "unknown gdr_status";
    }
}

}  // extern "C"

namespace {

// Validation shared by gdr_chunk_fwd and gdr_chunk_fwd_ws.  On success *launch tells whether
// there is work to enqueue and *BH is B * H.
gdr_status check_chunk(int64_t B, int64_t H, int64_t T, int d_k, int d_v, int io_dtype, int gate, const void* q,
                       const void* k, const void* v, const float* g, const float* beta, const float* initial_state,
                       const void* o, const float* final_state, int64_t* BHout, bool* launch) {
    *launch = false;
    if (B < 0 || H < 0 || T < 0) return GDR_ERR_INVALID_ARG;
    gdr_status s = check_common(d_k, d_v, io_dtype, gate);
    if (s != GDR_OK) return s;
    if (T > kMaxT) return GDR_ERR_SHAPE;
    int64_t BH, BHT, nq, nv, nstate, ng;
    const int64_t esz = io_dtype == GDR_BF16 ? 2 : 4;
    if (!mul_ok(B, H, &BH) || !mul_ok(BH, T, &BHT) || !mul_ok(BHT, d_k, &nq) || !mul_ok(BHT, d_v, &nv) ||
        !mul_ok(BH, (int64_t)d_k * d_v, &nstate) || !mul_ok(BHT, gate == GDR_GATE_CHANNEL ? d_k : 1, &ng) ||
        !mul_ok(nq, 4, &nq) || !mul_ok(nv, 4, &nv) || !mul_ok(nstate, 4, &nstate))
        return GDR_ERR_SHAPE;
    if (BHT > 0 && (!q || !k || !v || !g || !beta || !o)) return GDR_ERR_INVALID_ARG;
    // o must not overlap an input; the final state may alias the initial state exactly.
    const int64_t obytes = nv / 4 * esz, qbytes = nq / 4 * esz, vbytes = nv / 4 * esz;
    if (overlaps(o, obytes, q, qbytes) || overlaps(o, obytes, k, qbytes) || overlaps(o, obytes, v, vbytes) ||
        overlaps(o, obytes, initial_state, nstate) || overlaps(o, obytes, final_state, nstate))
        return GDR_ERR_INVALID_ARG;
    if (final_state && initial_state && final_state != initial_state &&
        overlaps(final_state, nstate, initial_state, nstate))
        return GDR_ERR_INVALID_ARG;
    if (io_dtype == GDR_F32 && (d_k != 64 || gate == GDR_GATE_CHANNEL)) return GDR_ERR_UNSUPPORTED;
    *BHout = BH;
    if (BH == 0) return GDR_OK;
    int64_t nwg;
    if (!mul_ok(BH, d_v / 32, &nwg) || nwg > kMaxGrid) return GDR_ERR_SHAPE;
    *launch = final_state != nullptr || BHT > 0;
    return GDR_OK;
}

hipError_t chunk_single_kernel(int64_t BH, int64_t T, int d_k, int d_v, int io_dtype, int gate, const void* q,
                               const void* k, const void* v, const float* g, const float* beta,
                               const float* initial_state, void* o, float* final_state, hipStream_t st) {
    if (io_dtype == GDR_BF16 && gate == GDR_GATE_CHANNEL)  // per-channel gate, fp16 MFMA
        return gdr::chunk_kda_dispatch(BH, T, d_k, d_v, q, k, v, g, beta, initial_state, o, final_state, st);
    if (io_dtype == GDR_BF16)  // fp16-MFMA producer/consumer kernel
        return gdr::chunk_fwd_pc_dispatch(BH, T, 1, d_k, d_v, q, k, v, g, beta, initial_state, o, final_state, st);
    // fp32 operands throughout
    return gdr::chunk_fwd_dispatch(BH, T, d_k, d_v, false, gate == GDR_GATE_CHANNEL, q, k, v, g, beta, initial_state,
                                   o, final_state, st);
}

// Workspace bytes of one sequence for the per-channel gate: the state kernel addresses it with
// 32-bit byte offsets.
int64_t kda_ws_bytes_per_seq(int64_t T, int d_k) {
    return (T + kChunkLen - 1) / kChunkLen * gdr::chunk_kda_ws_halfs(d_k) * 2;
}

// The two-kernel path serves bf16 I/O: the scalar gate always, the per-channel gate while one
// sequence's workspace stays below 4 GiB (T below about four million tokens).
bool uses_workspace(int64_t T, int d_k, int io_dtype, int gate) {
    if (io_dtype != GDR_BF16) return false;
    if (gate == GDR_GATE_SCALAR) return true;
    return kda_ws_bytes_per_seq(T, d_k) <= int64_t(0xffffffff);
}

}  // namespace

extern "C" {

gdr_status gdr_chunk_fwd(int64_t B, int64_t H, int64_t T, int d_k, int d_v, int io_dtype, int gate,
                         const void* q, const void* k, const void* v, const float* g, const float* beta,
                         const float* initial_state, void* o, float* final_state, void* stream) {
    int64_t BH = 0;
    bool launch = false;
    gdr_status s = check_chunk(B, H, T, d_k, d_v, io_dtype, gate, q, k, v, g, beta, initial_state, o, final_state,
                               &BH, &launch);
    if (s != GDR_OK || !launch) return s;
    hipError_t e = chunk_single_kernel(BH, T, d_k, d_v, io_dtype, gate, q, k, v, g, beta, initial_state, o,
                                       final_state, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

int64_t gdr_chunk_fwd_workspace_size(int64_t B, int64_t H, int64_t T, int d_k, int d_v, int io_dtype, int gate) {
    if (B < 0 || H < 0 || T < 0 || T > kMaxT) return -1;
    if (check_common(d_k, d_v, io_dtype, gate) != GDR_OK) return -1;
    int64_t BH, BHT, bytes;
    if (!mul_ok(B, H, &BH) || !mul_ok(BH, T + kChunkLen, &BHT) || !mul_ok(BHT, 4 * kChunkLen, &bytes)) return -1;
    if (!uses_workspace(T, d_k, io_dtype, gate)) return 0;
    if (gate == GDR_GATE_CHANNEL) return BH * kda_ws_bytes_per_seq(T, d_k);
    return gdr::chunk_split_workspace_bytes(BH, T);
}

gdr_status gdr_chunk_fwd_ws(int64_t B, int64_t H, int64_t T, int d_k, int d_v, int io_dtype, int gate,
                            const void* q, const void* k, const void* v, const float* g, const float* beta,
                            const float* initial_state, void* o, float* final_state, void* workspace,
                            int64_t workspace_bytes, void* stream) {
    int64_t BH = 0;
    bool launch = false;
    gdr_status s = check_chunk(B, H, T, d_k, d_v, io_dtype, gate, q, k, v, g, beta, initial_state, o, final_state,
                               &BH, &launch);
    if (s != GDR_OK) return s;
    if (workspace_bytes < 0) return GDR_ERR_INVALID_ARG;
    const int64_t need = gdr_chunk_fwd_workspace_size(B, H, T, d_k, d_v, io_dtype, gate);
    if (need < 0) return GDR_ERR_SHAPE;
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return GDR_ERR_INVALID_ARG;
    if (need > 0) {
        // the workspace is written by the first kernel: it may overlap no input and no output
        const int64_t esz = 2, BHT = BH * T, gw = gate == GDR_GATE_CHANNEL ? d_k : 1;
        if (overlaps(workspace, need, q, BHT * d_k * esz) || overlaps(workspace, need, k, BHT * d_k * esz) ||
            overlaps(workspace, need, v, BHT * d_v * esz) || overlaps(workspace, need, g, BHT * gw * 4) ||
            overlaps(workspace, need, beta, BHT * 4) || overlaps(workspace, need, o, BHT * d_v * esz) ||
            overlaps(workspace, need, initial_state, BH * d_k * d_v * 4) ||
            overlaps(workspace, need, final_state, BH * d_k * d_v * 4))
            return GDR_ERR_INVALID_ARG;
    }
    if (!launch) return GDR_OK;
    hipError_t e;
    if (need > 0 && gate == GDR_GATE_CHANNEL) {
        const hipStream_t st = static_cast<hipStream_t>(stream);
        e = gdr::chunk_kda_ut_dispatch(BH, T, d_k, q, k, g, beta, nullptr, workspace, st);
        if (e == hipSuccess)
            e = gdr::chunk_state_kda_dispatch(BH, T, d_k, d_v, v, nullptr, initial_state, o, final_state, workspace,
                                              st);
    } else if (need > 0)
        e = gdr::chunk_split_dispatch(BH, T, 1, d_k, d_v, q, k, v, g, beta, initial_state, o, final_state, workspace,
                                      static_cast<hipStream_t>(stream));
    else
        e = chunk_single_kernel(BH, T, d_k, d_v, io_dtype, gate, q, k, v, g, beta, initial_state, o, final_state,
                                static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

}  // extern "C"

namespace {

// Validation shared by gdr_gdp_chunk_fwd and gdr_gdp_chunk_fwd_ws.
gdr_status check_gdp(int64_t B, int64_t H, int64_t T, int n_h, int d_k, int d_v, int io_dtype, const void* q,
                     const void* k, const void* v, const float* g, const float* beta, const float* initial_state,
                     const void* o, const float* final_state, int64_t* BHout, bool* launch) {
    *launch = false;
    if (B < 0 || H < 0 || T < 0 || n_h < 1) return GDR_ERR_INVALID_ARG;
    gdr_status s = check_common(d_k, d_v, io_dtype, GDR_GATE_SCALAR);
    if (s != GDR_OK) return s;
    if (n_h > kMaxNh) return GDR_ERR_SHAPE;
    int64_t BH, BHT, BHTN, nq, nk, nv, no, nstate;
    if (!mul_ok(B, H, &BH) || !mul_ok(BH, T, &BHT) || !mul_ok(BHT, n_h, &BHTN) || !mul_ok(BHT, d_k, &nq) ||
        !mul_ok(BHTN, d_k, &nk) || !mul_ok(BHTN, d_v, &nv) || !mul_ok(BHT, d_v, &no) ||
        !mul_ok(BH, (int64_t)d_k * d_v, &nstate) || !mul_ok(nk, 4, &nk) || !mul_ok(nv, 4, &nv) ||
        !mul_ok(nstate, 4, &nstate))
        return GDR_ERR_SHAPE;
    if (T * n_h > kMaxT) return GDR_ERR_SHAPE;  // T <= kMaxT here, so the product fits
    if (BHT > 0 && (!q || !k || !v || !g || !beta || !o)) return GDR_ERR_INVALID_ARG;
    if (io_dtype != GDR_BF16) return GDR_ERR_UNSUPPORTED;
    // o must not overlap an input; the final state may alias the initial state exactly.
    const int64_t obytes = no * 2, qbytes = nq * 2, kbytes = nk / 2, vbytes = nv / 2;
    if (overlaps(o, obytes, q, qbytes) || overlaps(o, obytes, k, kbytes) || overlaps(o, obytes, v, vbytes) ||
        overlaps(o, obytes, g, BHT * 4) || overlaps(o, obytes, beta, BHTN * 4) ||
        overlaps(o, obytes, initial_state, nstate) || overlaps(o, obytes, final_state, nstate))
        return GDR_ERR_INVALID_ARG;
    if (final_state && initial_state && final_state != initial_state &&
        overlaps(final_state, nstate, initial_state, nstate))
        return GDR_ERR_INVALID_ARG;
    *BHout = BH;
    if (BH == 0) return GDR_OK;
    int64_t nwg;
    if (!mul_ok(BH, d_v / 32, &nwg) || nwg > kMaxGrid) return GDR_ERR_SHAPE;
    *launch = final_state != nullptr || BHT > 0;
    return GDR_OK;
}

}  // namespace

extern "C" {

gdr_status gdr_gdp_chunk_fwd(int64_t B, int64_t H, int64_t T, int n_h, int d_k, int d_v, int io_dtype,
                             const void* q, const void* k, const void* v, const float* g, const float* beta,
                             const float* initial_state, void* o, float* final_state, void* stream) {
    int64_t BH = 0;
    bool launch = false;
    gdr_status s = check_gdp(B, H, T, n_h, d_k, d_v, io_dtype, q, k, v, g, beta, initial_state, o, final_state, &BH,
                             &launch);
    if (s != GDR_OK || !launch) return s;
    hipError_t e = gdr::chunk_fwd_pc_dispatch(BH, T, n_h, d_k, d_v, q, k, v, g, beta, initial_state, o,
                                              final_state, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

int64_t gdr_gdp_chunk_fwd_workspace_size(int64_t B, int64_t H, int64_t T, int n_h, int d_k, int d_v) {
    if (B < 0 || H < 0 || T < 0 || n_h < 1 || n_h > kMaxNh || T > kMaxT || T * n_h > kMaxT) return -1;
    if (check_common(d_k, d_v, GDR_BF16, GDR_GATE_SCALAR) != GDR_OK) return -1;
    int64_t BH, x;
    if (!mul_ok(B, H, &BH) || !mul_ok(BH, T * n_h + kChunkLen, &x) || !mul_ok(x, 4 * kChunkLen, &x)) return -1;
    return gdr::chunk_split_workspace_bytes(BH, T * n_h);
}

gdr_status gdr_gdp_chunk_fwd_ws(int64_t B, int64_t H, int64_t T, int n_h, int d_k, int d_v, int io_dtype,
                                const void* q, const void* k, const void* v, const float* g, const float* beta,
                                const float* initial_state, void* o, float* final_state, void* workspace,
                                int64_t workspace_bytes, void* stream) {
    int64_t BH = 0;
    bool launch = false;
    gdr_status s = check_gdp(B, H, T, n_h, d_k, d_v, io_dtype, q, k, v, g, beta, initial_state, o, final_state, &BH,
                             &launch);
    if (s != GDR_OK) return s;
    if (workspace_bytes < 0) return GDR_ERR_INVALID_ARG;
    const int64_t need = gdr_gdp_chunk_fwd_workspace_size(B, H, T, n_h, d_k, d_v);
    if (need < 0) return GDR_ERR_SHAPE;
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return GDR_ERR_INVALID_ARG;
    if (need > 0) {
        // the workspace is written by the first kernel: it may overlap no input and no output
        const int64_t BHT = BH * T, BHTN = BHT * n_h;
        if (overlaps(workspace, need, q, BHT * d_k * 2) || overlaps(workspace, need, k, BHTN * d_k * 2) ||
            overlaps(workspace, need, v, BHTN * d_v * 2) || overlaps(workspace, need, g, BHT * 4) ||
            overlaps(workspace, need, beta, BHTN * 4) || overlaps(workspace, need, o, BHT * d_v * 2) ||
            overlaps(workspace, need, initial_state, BH * d_k * d_v * 4) ||
            overlaps(workspace, need, final_state, BH * d_k * d_v * 4))
            return GDR_ERR_INVALID_ARG;
    }
    if (!launch) return GDR_OK;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (need > 0)
        e = gdr::chunk_split_dispatch(BH, T, n_h, d_k, d_v, q, k, v, g, beta, initial_state, o, final_state, workspace,
                                      st);
    else
        e = gdr::chunk_fwd_pc_dispatch(BH, T, n_h, d_k, d_v, q, k, v, g, beta, initial_state, o, final_state, st);
    return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

}  // extern "C"

namespace {

// Validation shared by gdr_chunk_fwd_fused_prep and gdr_chunk_fwd_fused_prep_ws.
gdr_status check_prep(int64_t B, int64_t H, int64_t T, int d_k, int d_v, int io_dtype, const void* q_raw,
                      const void* k_raw, const void* v, const float* dt, const float* A_log, const float* dt_bias,
                      const float* beta_logit, const float* initial_state, const void* o, const float* final_state,
                      int64_t* BHout, bool* launch) {
    *launch = false;
    if (B < 0 || H < 0 || T < 0) return GDR_ERR_INVALID_ARG;
    gdr_status s = check_common(d_k, d_v, io_dtype, GDR_GATE_SCALAR);
    if (s != GDR_OK) return s;
    if (T > kMaxT) return GDR_ERR_SHAPE;
    int64_t BH, BHT, nq, nv, nstate;
    if (!mul_ok(B, H, &BH) || !mul_ok(BH, T, &BHT) || !mul_ok(BHT, d_k, &nq) || !mul_ok(BHT, d_v, &nv) ||
        !mul_ok(BH, (int64_t)d_k * d_v, &nstate) || !mul_ok(nq, 2, &nq) || !mul_ok(nv, 2, &nv) ||
        !mul_ok(nstate, 4, &nstate))
        return GDR_ERR_SHAPE;
    if (BHT > 0 && (!q_raw || !k_raw || !v || !dt || !beta_logit || !o)) return GDR_ERR_INVALID_ARG;
    if (BH > 0 && (!A_log || !dt_bias)) return GDR_ERR_INVALID_ARG;
    if (io_dtype != GDR_BF16) return GDR_ERR_UNSUPPORTED;
    // o must not overlap an input; the final state may alias the initial state exactly.
    if (overlaps(o, nv, q_raw, nq) || overlaps(o, nv, k_raw, nq) || overlaps(o, nv, v, nv) ||
        overlaps(o, nv, dt, BHT * 4) || overlaps(o, nv, beta_logit, BHT * 4) || overlaps(o, nv, A_log, H * 4) ||
        overlaps(o, nv, dt_bias, H * 4) || overlaps(o, nv, initial_state, nstate) ||
        overlaps(o, nv, final_state, nstate))
        return GDR_ERR_INVALID_ARG;
    if (final_state && initial_state && final_state != initial_state &&
        overlaps(final_state, nstate, initial_state, nstate))
        return GDR_ERR_INVALID_ARG;
    *BHout = BH;
    if (BH == 0) return GDR_OK;
    int64_t nwg;
    if (!mul_ok(BH, d_v / 32, &nwg) || nwg > kMaxGrid) return GDR_ERR_SHAPE;
    *launch = final_state != nullptr || BHT > 0;
    return GDR_OK;
}

}  // namespace

extern "C" {

gdr_status gdr_chunk_fwd_fused_prep(int64_t B, int64_t H, int64_t T, int d_k, int d_v, int io_dtype,
                                    const void* q_raw, const void* k_raw, const void* v, const float* dt,
                                    const float* A_log, const float* dt_bias, const float* beta_logit,
                                    const float* initial_state, void* o, float* final_state, void* stream) {
    int64_t BH = 0;
    bool launch = false;
    gdr_status s = check_prep(B, H, T, d_k, d_v, io_dtype, q_raw, k_raw, v, dt, A_log, dt_bias, beta_logit,
                              initial_state, o, final_state, &BH, &launch);
    if (s != GDR_OK || !launch) return s;
    hipError_t e = gdr::chunk_fwd_pc_prep_dispatch(BH, H, T, d_k, d_v, q_raw, k_raw, v, dt, A_log, dt_bias,
                                                   beta_logit, initial_state, o, final_state,
                                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

int64_t gdr_chunk_fwd_fused_prep_workspace_size(int64_t B, int64_t H, int64_t T, int d_k, int d_v) {
    if (B < 0 || H < 0 || T < 0 || T > kMaxT) return -1;
    if (check_common(d_k, d_v, GDR_BF16, GDR_GATE_SCALAR) != GDR_OK) return -1;
    int64_t BH, x;
    if (!mul_ok(B, H, &BH) || !mul_ok(BH, T + kChunkLen, &x) || !mul_ok(x, 4 * kChunkLen, &x)) return -1;
    return gdr::chunk_split_prep_workspace_bytes(BH, T, d_k);
}

gdr_status gdr_chunk_fwd_fused_prep_ws(int64_t B, int64_t H, int64_t T, int d_k, int d_v, int io_dtype,
                                       const void* q_raw, const void* k_raw, const void* v, const float* dt,
                                       const float* A_log, const float* dt_bias, const float* beta_logit,
                                       const float* initial_state, void* o, float* final_state, void* workspace,
                                       int64_t workspace_bytes, void* stream) {
    int64_t BH = 0;
    bool launch = false;
    gdr_status s = check_prep(B, H, T, d_k, d_v, io_dtype, q_raw, k_raw, v, dt, A_log, dt_bias, beta_logit,
                              initial_state, o, final_state, &BH, &launch);
    if (s != GDR_OK) return s;
    if (workspace_bytes < 0) return GDR_ERR_INVALID_ARG;
    const int64_t need = gdr_chunk_fwd_fused_prep_workspace_size(B, H, T, d_k, d_v);
    if (need < 0) return GDR_ERR_SHAPE;
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return GDR_ERR_INVALID_ARG;
    if (need > 0) {
        // the workspace is written by the first kernel: it may overlap no input and no output
        const int64_t BHT = BH * T;
        if (overlaps(workspace, need, q_raw, BHT * d_k * 2) || overlaps(workspace, need, k_raw, BHT * d_k * 2) ||
            overlaps(workspace, need, v, BHT * d_v * 2) || overlaps(workspace, need, dt, BHT * 4) ||
            overlaps(workspace, need, beta_logit, BHT * 4) || overlaps(workspace, need, A_log, H * 4) ||
            overlaps(workspace, need, dt_bias, H * 4) || overlaps(workspace, need, o, BHT * d_v * 2) ||
            overlaps(workspace, need, initial_state, BH * d_k * d_v * 4) ||
            overlaps(workspace, need, final_state, BH * d_k * d_v * 4))
            return GDR_ERR_INVALID_ARG;
    }
    if (!launch) return GDR_OK;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (need > 0)
        e = gdr::chunk_split_prep_dispatch(BH, H, T, d_k, d_v, q_raw, k_raw, v, dt, A_log, dt_bias, beta_logit,
                                           initial_state, o, final_state, workspace, st);
    else
        e = gdr::chunk_fwd_pc_prep_dispatch(BH, H, T, d_k, d_v, q_raw, k_raw, v, dt, A_log, dt_bias, beta_logit,
                                            initial_state, o, final_state, st);
    return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

}  // extern "C"

namespace {

// Validation shared by gdr_gdn2_chunk_fwd and gdr_gdn2_chunk_fwd_ws.
gdr_status check_gdn2(int64_t B, int64_t H, int64_t T, int d_k, int d_v, int io_dtype, const void* q, const void* k,
                      const void* v, const float* g, const float* b, const float* w, const float* initial_state,
                      const void* o, const float* final_state, int64_t* BHout, bool* launch) {
    *launch = false;
    if (B < 0 || H < 0 || T < 0) return GDR_ERR_INVALID_ARG;
    gdr_status s = check_common(d_k, d_v, io_dtype, GDR_GATE_CHANNEL);
    if (s != GDR_OK) return s;
    // the fp32 write gate is addressed with 32-bit byte offsets, one chunk past the end included
    if (T > kMaxT || (T + 64) * d_v > (int64_t(1) << 30)) return GDR_ERR_SHAPE;
    int64_t BH, BHT, nq, nv, nstate;
    if (!mul_ok(B, H, &BH) || !mul_ok(BH, T, &BHT) || !mul_ok(BHT, d_k, &nq) || !mul_ok(BHT, d_v, &nv) ||
        !mul_ok(BH, (int64_t)d_k * d_v, &nstate) || !mul_ok(nq, 4, &nq) || !mul_ok(nv, 4, &nv) ||
        !mul_ok(nstate, 4, &nstate))
        return GDR_ERR_SHAPE;
    if (BHT > 0 && (!q || !k || !v || !g || !b || !w || !o)) return GDR_ERR_INVALID_ARG;
    if (io_dtype != GDR_BF16) return GDR_ERR_UNSUPPORTED;
    // o must not overlap an input; the final state may alias the initial state exactly.
    const int64_t obytes = nv / 2, qbytes = nq / 2;
    if (overlaps(o, obytes, q, qbytes) || overlaps(o, obytes, k, qbytes) || overlaps(o, obytes, v, obytes) ||
        overlaps(o, obytes, g, nq) || overlaps(o, obytes, b, nq) || overlaps(o, obytes, w, nv) ||
        overlaps(o, obytes, initial_state, nstate) || overlaps(o, obytes, final_state, nstate))
        return GDR_ERR_INVALID_ARG;
    if (final_state && initial_state && final_state != initial_state &&
        overlaps(final_state, nstate, initial_state, nstate))
        return GDR_ERR_INVALID_ARG;
    *BHout = BH;
    if (BH == 0) return GDR_OK;
    int64_t nwg;
    if (!mul_ok(BH, d_v / 32, &nwg) || nwg > kMaxGrid) return GDR_ERR_SHAPE;
    *launch = final_state != nullptr || BHT > 0;
    return GDR_OK;
}

}  // namespace

extern "C" {

gdr_status gdr_gdn2_chunk_fwd(int64_t B, int64_t H, int64_t T, int d_k, int d_v, int io_dtype, const void* q,
                              const void* k, const void* v, const float* g, const float* b, const float* w,
                              const float* initial_state, void* o, float* final_state, void* stream) {
    int64_t BH = 0;
    bool launch = false;
    gdr_status s = check_gdn2(B, H, T, d_k, d_v, io_dtype, q, k, v, g, b, w, initial_state, o, final_state, &BH,
                              &launch);
    if (s != GDR_OK || !launch) return s;
    hipError_t e = gdr::chunk_gdn2_dispatch(BH, T, d_k, d_v, q, k, v, g, b, w, initial_state, o, final_state,
                                            static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

int64_t gdr_gdn2_chunk_fwd_workspace_size(int64_t B, int64_t H, int64_t T, int d_k, int d_v) {
    return gdr_chunk_fwd_workspace_size(B, H, T, d_k, d_v, GDR_BF16, GDR_GATE_CHANNEL);
}

gdr_status gdr_gdn2_chunk_fwd_ws(int64_t B, int64_t H, int64_t T, int d_k, int d_v, int io_dtype, const void* q,
                                 const void* k, const void* v, const float* g, const float* b, const float* w,
                                 const float* initial_state, void* o, float* final_state, void* workspace,
                                 int64_t workspace_bytes, void* stream) {
    int64_t BH = 0;
    bool launch = false;
    gdr_status s = check_gdn2(B, H, T, d_k, d_v, io_dtype, q, k, v, g, b, w, initial_state, o, final_state, &BH,
                              &launch);
    if (s != GDR_OK) return s;
    if (workspace_bytes < 0) return GDR_ERR_INVALID_ARG;
    const int64_t need = gdr_gdn2_chunk_fwd_workspace_size(B, H, T, d_k, d_v);
    if (need < 0) return GDR_ERR_SHAPE;
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return GDR_ERR_INVALID_ARG;
    if (need > 0) {
        // the workspace is written by the first kernel: it may overlap no input and no output
        const int64_t BHT = BH * T;
        if (overlaps(workspace, need, q, BHT * d_k * 2) || overlaps(workspace, need, k, BHT * d_k * 2) ||
            overlaps(workspace, need, v, BHT * d_v * 2) || overlaps(workspace, need, g, BHT * d_k * 4) ||
            overlaps(workspace, need, b, BHT * d_k * 4) || overlaps(workspace, need, w, BHT * d_v * 4) ||
            overlaps(workspace, need, o, BHT * d_v * 2) ||
            overlaps(workspace, need, initial_state, BH * d_k * d_v * 4) ||
            overlaps(workspace, need, final_state, BH * d_k * d_v * 4))
            return GDR_ERR_INVALID_ARG;
    }
    if (!launch) return GDR_OK;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (need > 0) {
        e = gdr::chunk_kda_ut_dispatch(BH, T, d_k, q, k, g, nullptr, b, workspace, st);
        if (e == hipSuccess)
            e = gdr::chunk_state_kda_dispatch(BH, T, d_k, d_v, v, w, initial_state, o, final_state, workspace, st);
    } else {
        e = gdr::chunk_gdn2_dispatch(BH, T, d_k, d_v, q, k, v, g, b, w, initial_state, o, final_state, st);
    }
    return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

int64_t gdr_frame_fwd_workspace_size(int64_t B, int64_t H, int64_t T, int frame_len, int d_k, int d_v) {
    if (B < 0 || H < 0 || T < 0 || T > kMaxT || frame_len < 16 || frame_len % 16 != 0) return -1;
    if ((d_k != 64 && d_k != 128) || (d_v != 64 && d_v != 128)) return -1;
    int64_t BH, x;
    const int64_t F = (T + frame_len - 1) / frame_len;
    if (!mul_ok(B, H, &BH) || !mul_ok(BH, F + 1, &x) || !mul_ok(x, 4 * 128 * 128 * 2, &x)) return -1;
    return gdr::frame_workspace_bytes(BH, T, frame_len, d_k, d_v);
}

gdr_status gdr_frame_fwd(int64_t B, int64_t H, int64_t T, int frame_len, int d_k, int d_v, int io_dtype, int gate,
                         const void* q, const void* k, const void* v, const float* gamma, const float* g,
                         const float* initial_state, void* o, float* final_state, void* workspace,
                         int64_t workspace_bytes, void* stream) {
    if (B < 0 || H < 0 || T < 0 || frame_len < 1) return GDR_ERR_INVALID_ARG;
    gdr_status s = check_common(d_k, d_v, io_dtype, gate);
    if (s != GDR_OK) return s;
    if (T > kMaxT || frame_len % 16 != 0) return GDR_ERR_SHAPE;
    if (io_dtype != GDR_BF16 || d_v == 32 || d_v > 128 || d_v == 96) return GDR_ERR_UNSUPPORTED;
    const int64_t F = (T + frame_len - 1) / frame_len;
    // the state pass addresses one sequence's W matrices with 32-bit byte offsets
    if ((F + 1) * d_k * d_k * 2 > (int64_t(1) << 31)) return GDR_ERR_SHAPE;
    int64_t BH, BHT, BHF, nq, nv, nstate, ng;
    if (!mul_ok(B, H, &BH) || !mul_ok(BH, T, &BHT) || !mul_ok(BH, F, &BHF) || !mul_ok(BHT, d_k * 2, &nq) ||
        !mul_ok(BHT, d_v * 2, &nv) || !mul_ok(BH, (int64_t)d_k * d_v * 4, &nstate) ||
        !mul_ok(BHF, gate == GDR_GATE_CHANNEL ? d_k * 4 : 4, &ng))
        return GDR_ERR_SHAPE;
    if (BHT > 0 && (!q || !k || !v || !gamma || !g || !o)) return GDR_ERR_INVALID_ARG;
    const int64_t need = gdr_frame_fwd_workspace_size(B, H, T, frame_len, d_k, d_v);
    if (need < 0) return GDR_ERR_SHAPE;
    if (workspace_bytes < 0 || (need > 0 && (!workspace || workspace_bytes < need))) return GDR_ERR_INVALID_ARG;
    if (overlaps(o, nv, q, nq) || overlaps(o, nv, k, nq) || overlaps(o, nv, v, nv) ||
        overlaps(o, nv, gamma, BHT * 4) || overlaps(o, nv, g, ng) || overlaps(o, nv, initial_state, nstate) ||
        overlaps(o, nv, final_state, nstate))
        return GDR_ERR_INVALID_ARG;
    if (final_state && initial_state && final_state != initial_state &&
        overlaps(final_state, nstate, initial_state, nstate))
        return GDR_ERR_INVALID_ARG;
    if (need > 0 &&
        (overlaps(workspace, need, q, nq) || overlaps(workspace, need, k, nq) || overlaps(workspace, need, v, nv) ||
         overlaps(workspace, need, gamma, BHT * 4) || overlaps(workspace, need, g, ng) ||
         overlaps(workspace, need, o, nv) || overlaps(workspace, need, initial_state, nstate) ||
         overlaps(workspace, need, final_state, nstate)))
        return GDR_ERR_INVALID_ARG;
    if (BH == 0) return GDR_OK;
    int64_t nwg;
    if (!mul_ok(BH, F > (T + 63) / 64 ? F : (T + 63) / 64, &nwg) || nwg > kMaxGrid) return GDR_ERR_SHAPE;
    if (!final_state && BHT == 0) return GDR_OK;
    hipError_t e = gdr::frame_dispatch(BH, T, frame_len, d_k, d_v, gate == GDR_GATE_CHANNEL, q, k, v, gamma, g,
                                       initial_state, o, final_state, workspace, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

gdr_status gdr_decode_step(int64_t N, int64_t H, int d_k, int d_v, int io_dtype, int gate, const void* q,
                           const void* k, const void* v, const float* g, const float* beta, float* state,
                           void* o, void* stream) {
    if (N < 0 || H < 0) return GDR_ERR_INVALID_ARG;
    gdr_status s = check_common(d_k, d_v, io_dtype, gate);
    if (s != GDR_OK) return s;
    int64_t NH, nstate;
    if (!mul_ok(N, H, &NH) || !mul_ok(NH, (int64_t)d_k * d_v, &nstate) || !mul_ok(nstate, 4, &nstate))
        return GDR_ERR_SHAPE;
    if (NH == 0) return GDR_OK;
    if (!q || !k || !v || !g || !beta || !state || !o) return GDR_ERR_INVALID_ARG;
    const int64_t esz = io_dtype == GDR_BF16 ? 2 : 4;
    const int64_t obytes = NH * d_v * esz;
    if (overlaps(o, obytes, state, nstate) || overlaps(o, obytes, q, NH * d_k * esz) ||
        overlaps(o, obytes, k, NH * d_k * esz) || overlaps(o, obytes, v, NH * d_v * esz))
        return GDR_ERR_INVALID_ARG;
    if (NH > kMaxGrid) return GDR_ERR_SHAPE;
    hipError_t e = gdr::decode_dispatch(NH, d_k, d_v, io_dtype == GDR_BF16, gate == GDR_GATE_CHANNEL, q, k, v, g,
                                        beta, state, o, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

}  // extern "C"
