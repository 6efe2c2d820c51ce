"""Write tests/golden/calibration_amax.json: the static global amax of every workload.

Calls only the CPU oracle (``oracle/``) and the seeded input generators
(``workloads/``).  The static activation amax plays the role of the calibrated
input amax of a static-NVFP4 Linear (FastVideo API page
``minimax_h3_nvfp4_fused``, NVFP4DecoderLinear with act_scale="static"; the
TensorRT-LLM fusions apply only to static NVFP4 scales).  For each workload:

  rms_adaln_256x2048     max |y| of the oracle's own modulated output y
  quantize_63240x7168    max |x| over 8,192 calibration rows (y = x)
  rms_adaln_63240x7168   max |y| of the oracle on 8,192 calibration rows,
  rms_adaln_300000x7168    frame index (r * T) // 8192
  swiglu_16384x19456     max |y| of the oracle on 2,048 calibration rows
  swiglu_bias_16384x19456, swiglu_paired_16384x19456
                         the same, with the workload's bias and column layout
  residual_rms_63240x7168  max |y| of the oracle (residual add, then RMSNorm) over
                         8,192 calibration rows of h and o
  residual_adaln_63240x7168  the same for the gated residual + RMSNorm + adaLN, frame
                         (r * 31) // 8192
  rms_silu_16x120x216x192  max |y| of the oracle over 32,768 calibration voxel rows
  ln_fp8_63240x7168      max |y| (fp32) of the oracle over 8,192 calibration rows; the
                         static FP8 scale is this amax / 448

Run:  python tests/golden/make_calibration.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402


def amax_of_bf16(u16) -> float:
    return float(np.max(np.abs(oracle.bf16_to_f32(u16))))


def calibrate(w: workloads.Workload) -> dict:
    if w.kind == "rms_adaln":
        if w.cal_rows == 0:
            x, idx, how = w.x(), w.frame_idx(), "max|y| of the oracle over the workload itself"
        else:
            x, idx = w.calibration_x(), w.calibration_frame_idx()
            how = "max|y| of the oracle over %d calibration rows" % w.cal_rows
        res = oracle.rms_adaln_rows(x, w.weight(), w.table(), idx, w.eps, 1.0, want_y=True)
        amax = amax_of_bf16(res["y"])
    elif w.kind == "quantize":
        amax = amax_of_bf16(w.calibration_x())
        how = "max|x| over %d calibration rows" % w.cal_rows
    elif w.kind == "ln_fp8":
        sc, sh = w.modulation()
        res = oracle.ln_adaln_fp8_rows(w.calibration_x(), sc, sh, w.eps, inv_scale=1.0)
        amax = float(np.abs(res["y"]).max())
        how = "max|y| of the oracle over %d calibration rows" % w.cal_rows
    elif w.kind == "rms_silu":
        res = oracle.rms_silu_rows(w.calibration_x(), w.weight(), w.eps, 1.0, want_y=True)
        amax = oracle.max_abs_f16(res["y"])
        how = "max|y| of the oracle over %d calibration rows" % w.cal_rows
    elif w.kind == "residual_adaln":
        res = oracle.residual_rms_adaln_rows(w.calibration_h(), w.calibration_o(), w.bias(), w.gate_table(),
                                             w.weight(), w.table(), w.calibration_frame_idx(), w.eps, 1.0,
                                             want_y=True)
        amax = amax_of_bf16(res["y"])
        how = "max|y| of the oracle over %d calibration rows" % w.cal_rows
    elif w.kind == "residual_rms":
        res = oracle.residual_rms_rows(w.calibration_h(), w.calibration_o(), w.bias(), w.residual_scale(),
                                       w.gamma(), w.eps, 1.0, want_y=True)
        amax = amax_of_bf16(res["y"])
        how = "max|y| of the oracle over %d calibration rows" % w.cal_rows
    elif w.kind == "swiglu" and (w.bias_std > 0 or w.interleaved):
        res = oracle.swiglu_packed_rows(w.calibration_x(), w.bias(), w.interleaved, 1.0, want_y=True)
        amax = amax_of_bf16(res["y"])
        how = "max|y| of the oracle over %d calibration rows" % w.cal_rows
    elif w.kind == "swiglu":
        o = w.calibration_x()
        res = oracle.swiglu_rows(o[:, :w.k], o[:, w.k:], 1.0, want_y=True)
        amax = amax_of_bf16(res["y"])
        how = "max|y| of the oracle over %d calibration rows" % w.cal_rows
    else:
        raise ValueError(w.kind)
    return {"global_amax": amax, "global_amax_hex": float(amax).hex(), "how": how}


def main():
    out = {}
    for name, w in workloads.WORKLOADS.items():
        out[name] = calibrate(w)
        print(name, out[name]["global_amax"], flush=True)
    path = os.path.join(ROOT, "tests", "golden", "calibration_amax.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
