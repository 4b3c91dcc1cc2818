"""Write tests/golden/bwd_rounding_model.json: the worst errors of the backward's rounding model
(tests/bwd_rounding_model.py: the oracle's exact gradients against the same gradients with the
roundings the algorithm cannot avoid) over the GPU backward tests' input cases. The GPU tests'
tolerances are a stated multiple of these figures; tests/test_bwd_tolerance_model.py recomputes them.

Run from the repository root: python tests/golden/make_bwd_rounding_model.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
sys.path.insert(0, os.path.dirname(HERE))

import bwd_rounding_model  # noqa: E402

if __name__ == "__main__":
    fig = bwd_rounding_model.model_figures()
    fig["note"] = ("worst |model - oracle| / (|oracle| + head rms) over dQ, dK, dV (elem_max) and worst "
                   "rms(model - oracle) / rms(oracle) per tensor (rms_max), over bwd_rounding_model.cases()")
    with open(os.path.join(HERE, "bwd_rounding_model.json"), "w") as f:
        json.dump(fig, f, indent=1)
        f.write("\n")
    print(fig)
