"""Writes ba_lm_traces.json: the oracle's LM traces on the seeded scenes.

Calls only ``oracle`` (its OpenMP build, which gives the plain build's bits,
as tests/test_oracle_threads.py pins) and ``synthetic``; no value comes from
the GPU library.  For every scene it records, per LM iteration, the cost
before and after the trial step, the decision, the damping used, the PCG
iteration count and relative residual, and the cost the state holds after the
iteration.  The iteration counts are those of the scenes' workloads: 20 on the
medium walk scene (with PCG, and with the dense reduced-camera solve,
"medium-dense"), 30 on the large scene (the 20-iteration trace that the
benchmark times is its prefix), 20 on the wide scene.

    python tests/golden/make_ba_traces.py            # all scenes
    python tests/golden/make_ba_traces.py medium     # one scene
"""
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from synthetic import ba_scene  # noqa: E402

OUT = os.path.join(HERE, "ba_lm_traces.json")
RUNS = {"medium": 20, "large": 30, "wide": 20, "medium-dense": 20}


def trace(name, n_iters):
    config, _, solver = name.partition("-")
    sc = ba_scene(config)
    P = oracle.Problem.from_scene(sc, parallel=True, solver=1 if solver == "dense" else 0)
    steps = []
    for _ in range(n_iters):
        s = P.lm_step()
        steps.append({"cost_before": s["cost_before"], "cost_after": s["cost_after"],
                      "accepted": s["accepted"], "lam": s["lam"], "pcg_iters": s["pcg_iters"],
                      "pcg_rel_res": s["pcg_rel_res"], "cost": P.cost})
    return {"solver": "dense" if solver == "dense" else "pcg", "n_obs": len(sc["obs_cam"]), "n_pts": len(sc["points"]), "n_cams": len(sc["cams"]),
            "loss": sc["loss"], "pcg_max_iters": sc["pcg_max_iters"],
            "pcg_rel_tol": sc["pcg_rel_tol"], "seed": sc["seed"], "steps": steps}


def main(names):
    data = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            data = json.load(f)
    for name in names:
        t0 = time.time()
        data[name] = trace(name, RUNS[name])
        print(f"{name}: {RUNS[name]} LM iterations in {time.time() - t0:.1f} s, final cost "
              f"{data[name]['steps'][-1]['cost']!r} ({oracle.num_threads(True)} threads)",
              flush=True)
    data["_source"] = ("oracle LM traces (tests/golden/make_ba_traces.py); scenes from "
                       "synthetic.ba_scene with their default seeds")
    with open(OUT, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:] or list(RUNS))
