"""Error measures for GPU-vs-oracle parity (shared by the GPU tests and the bench).

* literal:   max_i |x_i - ref_i| / RMS(ref)                 (fp32 outputs, the state)
* bf16 out:  max_i (|x_i - ref_i| - 2^-8 max(|x_i|, |ref_i|))_+ / RMS(ref)
             -- a bf16 output is charged only beyond its own final rounding (an output
             rounded to bf16 can be off by up to 2^-8 relative even when exact before).
Bars: 2e-2 for bf16 I/O, 1e-4 for fp32 I/O, applied to o and to the final state.
"""
import numpy as np

TOL_BF16 = 2e-2
TOL_F32 = 1e-4


def rms(ref):
    return float(np.sqrt(np.mean(np.asarray(ref, dtype=np.float64) ** 2)))


def err_literal(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(x - ref))) / max(rms(ref), 1e-30)


def err_bf16_out(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(x - ref) - 2.0 ** -8 * np.maximum(np.abs(x), np.abs(ref))
    return float(np.max(np.maximum(d, 0.0))) / max(rms(ref), 1e-30)


def bf16_floor(ref):
    """max |bf16(ref) - ref| / RMS(ref): what rounding the exact output alone costs."""
    import gdr_synth
    r32 = np.asarray(ref, dtype=np.float32)
    return err_literal(gdr_synth.round_to_bf16(r32).astype(np.float64), ref)


def report(name, o, o_ref, S, S_ref, bf16):
    eo = err_bf16_out(o, o_ref) if bf16 else err_literal(o, o_ref)
    es = err_literal(S, S_ref) if S is not None else 0.0
    msg = f"{name}: e_o={eo:.3e} e_S={es:.3e}"
    if bf16:
        msg += f" raw_o={err_literal(o, o_ref):.3e} floor_o={bf16_floor(o_ref):.3e}"
    return eo, es, msg
