// gdr_api.hip -- host side of the libgdr C ABI: argument validation and kernel dispatch.
// Declarations and the contract of every entry point are in include/gdr.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "gdr.h"

namespace gdr {
hipError_t chunk_fwd_f32_dispatch(int64_t BH, int64_t T, int dv, const void* q, const void* k, const void* v,
                                  const float* g, const float* beta, const float* S0, void* o, float* Sf,
                                  hipStream_t st);
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
hipError_t frame_dispatch(int64_t BH, int64_t T, int n, int dk, int dv, bool channel, const void* q, const void* k,
                          const void* v, const float* gamma, const float* g, const float* S0, void* o, float* Sf,
                          void* ws, hipStream_t st);
int64_t frame_workspace_bytes(int64_t BH, int64_t T, int n, int dk, int dv);
hipError_t decode_dispatch(int64_t NH, int dk, int dv, bool bf16, bool channel, const void* q, const void* k,
                           const void* v, const float* g, const float* beta, float* S, void* o, hipStream_t st);
}  // namespace gdr

namespace {

constexpr int kVersion = 10000 * 0 + 100 * 2 + 0;
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

// One buffer of a call, for the overlap checks: base pointer and size in bytes.
struct Span {
    const void* p;
    int64_t n;
};

// The workspace of a call: at least `need` bytes (need > 0), and overlapping none of the
// call's buffers.  need == 0: the workspace is ignored.
gdr_status check_workspace(const void* ws, int64_t bytes, int64_t need, const Span* bufs, int nbufs) {
    if (bytes < 0) return GDR_ERR_WORKSPACE;
    if (need <= 0) return GDR_OK;
    if (ws == nullptr || bytes < need) return GDR_ERR_WORKSPACE;
    for (int i = 0; i < nbufs; ++i)
        if (overlaps(ws, need, bufs[i].p, bufs[i].n)) return GDR_ERR_WORKSPACE;
    return GDR_OK;
}

// The output o may overlap none of the inputs; the final state may alias the initial state
// exactly but overlap it no other way.
gdr_status check_aliasing(const void* o, int64_t obytes, const Span* ins, int nins, const float* S0,
                          const float* Sf, int64_t sbytes) {
    for (int i = 0; i < nins; ++i)
        if (overlaps(o, obytes, ins[i].p, ins[i].n)) return GDR_ERR_INVALID_ARG;
    if (overlaps(o, obytes, S0, sbytes) || overlaps(o, obytes, Sf, sbytes)) return GDR_ERR_INVALID_ARG;
    if (Sf && S0 && Sf != S0 && overlaps(Sf, sbytes, S0, sbytes)) return GDR_ERR_INVALID_ARG;
    return GDR_OK;
}

gdr_status from_hip(hipError_t e) { return e == hipSuccess ? GDR_OK : GDR_ERR_HIP; }

// Both grids of a chunked call fit a launch: the state pass's B*H*d_v/16 groups (at most) and
// the UT pass's B*H*ceil(steps/64) (one group per chunk).
bool grids_ok(int64_t BH, int d_v, int64_t steps) {
    int64_t a = 0, b = 0;
    return mul_ok(BH, d_v / 16, &a) && a <= kMaxGrid && mul_ok(BH, (steps + kChunkLen - 1) / kChunkLen, &b) &&
           b <= kMaxGrid;
}

// Per-channel workspace bytes of one sequence: the state kernel addresses them with 32-bit
// offsets, so they must stay below 4 GiB.
int64_t kda_ws_bytes_per_seq(int64_t T, int d_k) {
    return (T + kChunkLen - 1) / kChunkLen * gdr::chunk_kda_ws_halfs(d_k) * 2;
}

}  // namespace

extern "C" {

int gdr_version(void) { return kVersion; }

const char* gdr_status_string(int status) {
    switch (status) {
        case GDR_OK: return "success";
        case GDR_ERR_INVALID_ARG: return "invalid argument (null buffer, negative size, bad enum or overlapping output)";
        case GDR_ERR_SHAPE: return "unsupported size (d_k must be 64 or 128, d_v a multiple of 32 in [32, 256])";
        case GDR_ERR_DTYPE: return "unsupported io dtype (GDR_BF16 or GDR_F32)";
        case GDR_ERR_UNSUPPORTED: return "valid but unsupported combination of arguments";
        case GDR_ERR_WORKSPACE: return "workspace missing, too small, or overlapping an input or output";
        case GDR_ERR_HIP: return "HIP runtime error while enqueuing the kernel";
        default: return "unknown gdr_status";
    }
}

}  // extern "C"

namespace {

// Validation of gdr_chunk_fwd's tensor arguments.  On success *launch tells whether there is
// work to enqueue and *BH is B * H.
gdr_status check_chunk(int64_t B, int64_t H, int64_t T, int d_k, int d_v, int io_dtype, int gate, const void* q,
                       const void* k, const void* v, const float* g, const float* beta, const float* initial_state,
                       const void* o, const float* final_state, int64_t* BHout, bool* launch) {
    *launch = false;
    if (B < 0 || H < 0 || T < 0) return GDR_ERR_INVALID_ARG;
    gdr_status s = check_common(d_k, d_v, io_dtype, gate);
    if (s != GDR_OK) return s;
    if (T > kMaxT) return GDR_ERR_SHAPE;
    if (gate == GDR_GATE_CHANNEL && kda_ws_bytes_per_seq(T, d_k) > int64_t(0xffffffff)) return GDR_ERR_SHAPE;
    int64_t BH, BHT, nq, nv, nstate, ng;
    const int64_t esz = io_dtype == GDR_BF16 ? 2 : 4;
    if (!mul_ok(B, H, &BH) || !mul_ok(BH, T, &BHT) || !mul_ok(BHT, d_k, &nq) || !mul_ok(BHT, d_v, &nv) ||
        !mul_ok(BH, (int64_t)d_k * d_v, &nstate) || !mul_ok(BHT, gate == GDR_GATE_CHANNEL ? d_k : 1, &ng) ||
        !mul_ok(nq, 4, &nq) || !mul_ok(nv, 4, &nv) || !mul_ok(nstate, 4, &nstate) || !mul_ok(ng, 4, &ng))
        return GDR_ERR_SHAPE;
    if (BHT > 0 && (!q || !k || !v || !g || !beta || !o)) return GDR_ERR_INVALID_ARG;
    const int64_t qbytes = nq / 4 * esz, vbytes = nv / 4 * esz;
    const Span ins[] = {{q, qbytes}, {k, qbytes}, {v, vbytes}, {g, ng}, {beta, BHT * 4}};
    s = check_aliasing(o, vbytes, ins, 5, initial_state, final_state, nstate);
    if (s != GDR_OK) return s;
    if (io_dtype == GDR_F32 && (d_k != 64 || gate == GDR_GATE_CHANNEL)) return GDR_ERR_UNSUPPORTED;
    *BHout = BH;
    if (BH == 0) return GDR_OK;
    if (!grids_ok(BH, d_v, T)) return GDR_ERR_SHAPE;
    *launch = final_state != nullptr || BHT > 0;
    return GDR_OK;
}

// The kernels of gdr_chunk_fwd on validated arguments and a workspace of the required size.
gdr_status enqueue_chunk(int64_t BH, int64_t T, int d_k, int d_v, int io_dtype, int gate, const void* q, const void* k,
                         const void* v, const float* g, const float* beta, const float* initial_state, void* o,
                         float* final_state, void* workspace, hipStream_t st) {
    if (io_dtype == GDR_F32)  // fp32 operands throughout, one kernel
        return from_hip(gdr::chunk_fwd_f32_dispatch(BH, T, d_v, q, k, v, g, beta, initial_state, o, final_state, st));
    if (gate == GDR_GATE_CHANNEL) {
        hipError_t e = gdr::chunk_kda_ut_dispatch(BH, T, d_k, q, k, g, beta, nullptr, workspace, st);
        if (e == hipSuccess)
            e = gdr::chunk_state_kda_dispatch(BH, T, d_k, d_v, v, nullptr, initial_state, o, final_state, workspace,
                                              st);
        return from_hip(e);
    }
    return from_hip(gdr::chunk_split_dispatch(BH, T, 1, d_k, d_v, q, k, v, g, beta, initial_state, o, final_state,
                                              workspace, st));
}

}  // namespace

extern "C" {

int64_t gdr_chunk_fwd_workspace_size(int64_t B, int64_t H, int64_t T, int d_k, int d_v, int io_dtype, int gate) {
    if (B < 0 || H < 0 || T < 0 || T > kMaxT) return -1;
    if (check_common(d_k, d_v, io_dtype, gate) != GDR_OK) return -1;
    int64_t BH, BHT, bytes;
    if (!mul_ok(B, H, &BH) || !mul_ok(BH, T + kChunkLen, &BHT) || !mul_ok(BHT, 4 * kChunkLen, &bytes)) return -1;
    if (io_dtype == GDR_F32) return (d_k == 64 && gate == GDR_GATE_SCALAR) ? 0 : -1;  // one kernel, no workspace
    if (gate == GDR_GATE_CHANNEL) {
        const int64_t per = kda_ws_bytes_per_seq(T, d_k);
        return per > int64_t(0xffffffff) ? -1 : BH * per;
    }
    return gdr::chunk_split_workspace_bytes(BH, T);
}

gdr_status gdr_chunk_fwd(int64_t B, int64_t H, int64_t T, int d_k, int d_v, int io_dtype, int gate,
                         const void* q, const void* k, const void* v, const float* g, const float* beta,
                         const float* initial_state, void* o, float* final_state, void* workspace,
                         int64_t workspace_bytes, void* stream) {
    int64_t BH = 0;
    bool launch = false;
    gdr_status s = check_chunk(B, H, T, d_k, d_v, io_dtype, gate, q, k, v, g, beta, initial_state, o, final_state,
                               &BH, &launch);
    if (s != GDR_OK) return s;
    const int64_t need = gdr_chunk_fwd_workspace_size(B, H, T, d_k, d_v, io_dtype, gate);
    if (need < 0) return GDR_ERR_SHAPE;
    const int64_t esz = io_dtype == GDR_BF16 ? 2 : 4, BHT = BH * T, gw = gate == GDR_GATE_CHANNEL ? d_k : 1;
    const Span bufs[] = {{q, BHT * d_k * esz},         {k, BHT * d_k * esz},         {v, BHT * d_v * esz},
                         {g, BHT * gw * 4},            {beta, BHT * 4},              {o, BHT * d_v * esz},
                         {initial_state, BH * d_k * d_v * 4}, {final_state, BH * d_k * d_v * 4}};
    s = check_workspace(workspace, workspace_bytes, need, bufs, 8);
    if (s != GDR_OK || !launch) return s;
    return enqueue_chunk(BH, T, d_k, d_v, io_dtype, gate, q, k, v, g, beta, initial_state, o, final_state, workspace,
                         static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// Validation of gdr_gdp_chunk_fwd's tensor arguments.
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
    const Span ins[] = {{q, nq * 2}, {k, nk / 2}, {v, nv / 2}, {g, BHT * 4}, {beta, BHTN * 4}};
    s = check_aliasing(o, no * 2, ins, 5, initial_state, final_state, nstate);
    if (s != GDR_OK) return s;
    *BHout = BH;
    if (BH == 0) return GDR_OK;
    if (!grids_ok(BH, d_v, T * n_h)) return GDR_ERR_SHAPE;
    *launch = final_state != nullptr || BHT > 0;
    return GDR_OK;
}

}  // namespace

extern "C" {

int64_t gdr_gdp_chunk_fwd_workspace_size(int64_t B, int64_t H, int64_t T, int n_h, int d_k, int d_v) {
    if (B < 0 || H < 0 || T < 0 || n_h < 1 || n_h > kMaxNh || T > kMaxT || T * n_h > kMaxT) return -1;
    if (check_common(d_k, d_v, GDR_BF16, GDR_GATE_SCALAR) != GDR_OK) return -1;
    int64_t BH, x;
    if (!mul_ok(B, H, &BH) || !mul_ok(BH, T * n_h + kChunkLen, &x) || !mul_ok(x, 4 * kChunkLen, &x)) return -1;
    return gdr::chunk_split_workspace_bytes(BH, T * n_h);
}

gdr_status gdr_gdp_chunk_fwd(int64_t B, int64_t H, int64_t T, int n_h, int d_k, int d_v, int io_dtype,
                             const void* q, const void* k, const void* v, const float* g, const float* beta,
                             const float* initial_state, void* o, float* final_state, void* workspace,
                             int64_t workspace_bytes, void* stream) {
    int64_t BH = 0;
    bool launch = false;
    gdr_status s = check_gdp(B, H, T, n_h, d_k, d_v, io_dtype, q, k, v, g, beta, initial_state, o, final_state, &BH,
                             &launch);
    if (s != GDR_OK) return s;
    const int64_t need = gdr_gdp_chunk_fwd_workspace_size(B, H, T, n_h, d_k, d_v);
    if (need < 0) return GDR_ERR_SHAPE;
    const int64_t BHT = BH * T, BHTN = BHT * n_h;
    const Span bufs[] = {{q, BHT * d_k * 2},   {k, BHTN * d_k * 2}, {v, BHTN * d_v * 2},
                         {g, BHT * 4},          {beta, BHTN * 4},    {o, BHT * d_v * 2},
                         {initial_state, BH * d_k * d_v * 4}, {final_state, BH * d_k * d_v * 4}};
    s = check_workspace(workspace, workspace_bytes, need, bufs, 8);
    if (s != GDR_OK || !launch) return s;
    return from_hip(gdr::chunk_split_dispatch(BH, T, n_h, d_k, d_v, q, k, v, g, beta, initial_state, o, final_state,
                                              workspace, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Validation of gdr_chunk_fwd_fused_prep's tensor arguments.
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
    const Span ins[] = {{q_raw, nq}, {k_raw, nq}, {v, nv}, {dt, BHT * 4}, {beta_logit, BHT * 4},
                        {A_log, H * 4}, {dt_bias, H * 4}};
    s = check_aliasing(o, nv, ins, 7, initial_state, final_state, nstate);
    if (s != GDR_OK) return s;
    *BHout = BH;
    if (BH == 0) return GDR_OK;
    if (!grids_ok(BH, d_v, T)) return GDR_ERR_SHAPE;
    *launch = final_state != nullptr || BHT > 0;
    return GDR_OK;
}

}  // namespace

extern "C" {

int64_t gdr_chunk_fwd_fused_prep_workspace_size(int64_t B, int64_t H, int64_t T, int d_k, int d_v) {
    if (B < 0 || H < 0 || T < 0 || T > kMaxT) return -1;
    if (check_common(d_k, d_v, GDR_BF16, GDR_GATE_SCALAR) != GDR_OK) return -1;
    int64_t BH, x;
    if (!mul_ok(B, H, &BH) || !mul_ok(BH, T + kChunkLen, &x) || !mul_ok(x, 4 * kChunkLen, &x)) return -1;
    return gdr::chunk_split_prep_workspace_bytes(BH, T, d_k);
}

gdr_status gdr_chunk_fwd_fused_prep(int64_t B, int64_t H, int64_t T, int d_k, int d_v, int io_dtype,
                                    const void* q_raw, const void* k_raw, const void* v, const float* dt,
                                    const float* A_log, const float* dt_bias, const float* beta_logit,
                                    const float* initial_state, void* o, float* final_state, void* workspace,
                                    int64_t workspace_bytes, void* stream) {
    int64_t BH = 0;
    bool launch = false;
    gdr_status s = check_prep(B, H, T, d_k, d_v, io_dtype, q_raw, k_raw, v, dt, A_log, dt_bias, beta_logit,
                              initial_state, o, final_state, &BH, &launch);
    if (s != GDR_OK) return s;
    const int64_t need = gdr_chunk_fwd_fused_prep_workspace_size(B, H, T, d_k, d_v);
    if (need < 0) return GDR_ERR_SHAPE;
    const int64_t BHT = BH * T;
    const Span bufs[] = {{q_raw, BHT * d_k * 2}, {k_raw, BHT * d_k * 2}, {v, BHT * d_v * 2},
                         {dt, BHT * 4},          {beta_logit, BHT * 4},  {A_log, H * 4},
                         {dt_bias, H * 4},       {o, BHT * d_v * 2},     {initial_state, BH * d_k * d_v * 4},
                         {final_state, BH * d_k * d_v * 4}};
    s = check_workspace(workspace, workspace_bytes, need, bufs, 10);
    if (s != GDR_OK || !launch) return s;
    return from_hip(gdr::chunk_split_prep_dispatch(BH, H, T, d_k, d_v, q_raw, k_raw, v, dt, A_log, dt_bias,
                                                   beta_logit, initial_state, o, final_state, workspace,
                                                   static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Validation of gdr_gdn2_chunk_fwd's tensor arguments.
gdr_status check_gdn2(int64_t B, int64_t H, int64_t T, int d_k, int d_v, int io_dtype, const void* q, const void* k,
                      const void* v, const float* g, const float* b, const float* w, const float* initial_state,
                      const void* o, const float* final_state, int64_t* BHout, bool* launch) {
    *launch = false;
    if (B < 0 || H < 0 || T < 0) return GDR_ERR_INVALID_ARG;
    gdr_status s = check_common(d_k, d_v, io_dtype, GDR_GATE_CHANNEL);
    if (s != GDR_OK) return s;
    // the fp32 write gate is addressed with 32-bit byte offsets, one chunk past the end included
    if (T > kMaxT || (T + 64) * d_v > (int64_t(1) << 30)) return GDR_ERR_SHAPE;
    if (kda_ws_bytes_per_seq(T, d_k) > int64_t(0xffffffff)) return GDR_ERR_SHAPE;
    int64_t BH, BHT, nq, nv, nstate;
    if (!mul_ok(B, H, &BH) || !mul_ok(BH, T, &BHT) || !mul_ok(BHT, d_k, &nq) || !mul_ok(BHT, d_v, &nv) ||
        !mul_ok(BH, (int64_t)d_k * d_v, &nstate) || !mul_ok(nq, 4, &nq) || !mul_ok(nv, 4, &nv) ||
        !mul_ok(nstate, 4, &nstate))
        return GDR_ERR_SHAPE;
    if (BHT > 0 && (!q || !k || !v || !g || !b || !w || !o)) return GDR_ERR_INVALID_ARG;
    if (io_dtype != GDR_BF16) return GDR_ERR_UNSUPPORTED;
    const Span ins[] = {{q, nq / 2}, {k, nq / 2}, {v, nv / 2}, {g, nq}, {b, nq}, {w, nv}};
    s = check_aliasing(o, nv / 2, ins, 6, initial_state, final_state, nstate);
    if (s != GDR_OK) return s;
    *BHout = BH;
    if (BH == 0) return GDR_OK;
    if (!grids_ok(BH, d_v, T)) return GDR_ERR_SHAPE;
    *launch = final_state != nullptr || BHT > 0;
    return GDR_OK;
}

}  // namespace

extern "C" {

int64_t gdr_gdn2_chunk_fwd_workspace_size(int64_t B, int64_t H, int64_t T, int d_k, int d_v) {
    return gdr_chunk_fwd_workspace_size(B, H, T, d_k, d_v, GDR_BF16, GDR_GATE_CHANNEL);
}

gdr_status gdr_gdn2_chunk_fwd(int64_t B, int64_t H, int64_t T, int d_k, int d_v, int io_dtype, const void* q,
                              const void* k, const void* v, const float* g, const float* b, const float* w,
                              const float* initial_state, void* o, float* final_state, void* workspace,
                              int64_t workspace_bytes, void* stream) {
    int64_t BH = 0;
    bool launch = false;
    gdr_status s = check_gdn2(B, H, T, d_k, d_v, io_dtype, q, k, v, g, b, w, initial_state, o, final_state, &BH,
                              &launch);
    if (s != GDR_OK) return s;
    const int64_t need = gdr_gdn2_chunk_fwd_workspace_size(B, H, T, d_k, d_v);
    if (need < 0) return GDR_ERR_SHAPE;
    const int64_t BHT = BH * T;
    const Span bufs[] = {{q, BHT * d_k * 2}, {k, BHT * d_k * 2}, {v, BHT * d_v * 2},
                         {g, BHT * d_k * 4}, {b, BHT * d_k * 4}, {w, BHT * d_v * 4},
                         {o, BHT * d_v * 2}, {initial_state, BH * d_k * d_v * 4}, {final_state, BH * d_k * d_v * 4}};
    s = check_workspace(workspace, workspace_bytes, need, bufs, 9);
    if (s != GDR_OK || !launch) return s;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = gdr::chunk_kda_ut_dispatch(BH, T, d_k, q, k, g, nullptr, b, workspace, st);
    if (e == hipSuccess)
        e = gdr::chunk_state_kda_dispatch(BH, T, d_k, d_v, v, w, initial_state, o, final_state, workspace, st);
    return from_hip(e);
}

int64_t gdr_frame_fwd_workspace_size(int64_t B, int64_t H, int64_t T, int frame_len, int d_k, int d_v) {
    if (B < 0 || H < 0 || T < 0 || T > kMaxT || frame_len < 16 || frame_len % 16 != 0) return -1;
    if ((d_k != 64 && d_k != 128) || (d_v != 64 && d_v != 128)) return -1;
    const int64_t F = (T + frame_len - 1) / frame_len;
    // the state pass addresses one sequence's W, C and state records with 32-bit byte offsets
    // (one frame past the end included)
    if ((F + 1) * (int64_t)d_v * d_k * 4 > int64_t(0xffffffff)) return -1;
    int64_t BH, x;
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
    int64_t BH, BHT, BHF, nq, nv, nstate, ng;
    if (!mul_ok(B, H, &BH) || !mul_ok(BH, T, &BHT) || !mul_ok(BH, F, &BHF) || !mul_ok(BHT, d_k * 2, &nq) ||
        !mul_ok(BHT, d_v * 2, &nv) || !mul_ok(BH, (int64_t)d_k * d_v * 4, &nstate) ||
        !mul_ok(BHF, gate == GDR_GATE_CHANNEL ? d_k * 4 : 4, &ng))
        return GDR_ERR_SHAPE;
    const int64_t need = gdr_frame_fwd_workspace_size(B, H, T, frame_len, d_k, d_v);
    if (need < 0) return GDR_ERR_SHAPE;
    if (BHT > 0 && (!q || !k || !v || !gamma || !g || !o)) return GDR_ERR_INVALID_ARG;
    const Span ins[] = {{q, nq}, {k, nq}, {v, nv}, {gamma, BHT * 4}, {g, ng}};
    s = check_aliasing(o, nv, ins, 5, initial_state, final_state, nstate);
    if (s != GDR_OK) return s;
    const Span bufs[] = {{q, nq}, {k, nq}, {v, nv}, {gamma, BHT * 4}, {g, ng}, {o, nv},
                         {initial_state, nstate}, {final_state, nstate}};
    s = check_workspace(workspace, workspace_bytes, need, bufs, 8);
    if (s != GDR_OK) return s;
    if (BH == 0) return GDR_OK;
    int64_t nwg;
    if (!mul_ok(BH, F > (T + 63) / 64 ? F : (T + 63) / 64, &nwg) || nwg > kMaxGrid) return GDR_ERR_SHAPE;
    if (!final_state && BHT == 0) return GDR_OK;
    return from_hip(gdr::frame_dispatch(BH, T, frame_len, d_k, d_v, gate == GDR_GATE_CHANNEL, q, k, v, gamma, g,
                                        initial_state, o, final_state, workspace, static_cast<hipStream_t>(stream)));
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
    return from_hip(gdr::decode_dispatch(NH, d_k, d_v, io_dtype == GDR_BF16, gate == GDR_GATE_CHANNEL, q, k, v, g,
                                         beta, state, o, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// gdr_chunk_fwd_noalloc: gdr_chunk_fwd with the library's own device workspace, for callers that
// cannot allocate.  The workspace is this file-scope array: every GPU the library runs on holds
// one copy, from module load until the process ends.  Host code never uses the array's name
// as an address (on the host it only names the symbol); the device address of each GPU's copy
// comes from hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[GDR_CHUNK_FWD_NOALLOC_WORKSPACE_BYTES];

namespace {

std::atomic<void*> g_scratch[64];  // device address of `scratch`, per device id below 64

hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool slot = dev >= 0 && dev < 64;
    if (slot) {
        void* p = g_scratch[dev].load(std::memory_order_acquire);
        if (p != nullptr) {
            *out = p;
            return hipSuccess;
        }
    }
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    if (slot) g_scratch[dev].store(p, std::memory_order_release);  // concurrent first calls store the same value
    *out = p;
    return hipSuccess;
}

}  // namespace

extern "C" {

gdr_status gdr_chunk_fwd_noalloc(int64_t B, int64_t H, int64_t T, int d_k, int d_v, int io_dtype, int gate,
                                 const void* q, const void* k, const void* v, const float* g, const float* beta,
                                 const float* initial_state, void* o, float* final_state, void* stream) {
    int64_t BH = 0;
    bool launch = false;
    gdr_status s = check_chunk(B, H, T, d_k, d_v, io_dtype, gate, q, k, v, g, beta, initial_state, o, final_state,
                               &BH, &launch);
    if (s != GDR_OK) return s;
    const int64_t need = gdr_chunk_fwd_workspace_size(B, H, T, d_k, d_v, io_dtype, gate);
    if (need < 0) return GDR_ERR_SHAPE;
    if (need > (int64_t)GDR_CHUNK_FWD_NOALLOC_WORKSPACE_BYTES) return GDR_ERR_WORKSPACE;
    if (!launch) return GDR_OK;
    void* ws = nullptr;
    if (need > 0 && scratch_address(&ws) != hipSuccess) return GDR_ERR_HIP;
    return enqueue_chunk(BH, T, d_k, d_v, io_dtype, gate, q, k, v, g, beta, initial_state, o, final_state, ws,
                         static_cast<hipStream_t>(stream));
}

}  // extern "C"
