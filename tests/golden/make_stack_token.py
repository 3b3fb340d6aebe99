"""Pick the activation draw used by the 8-layer stack test (oracle only).

Writes stack8_token.json: the first draw of the k3_stack8 workload whose
fp64 oracle chain has a k-th/(k+1)-th router-logit gap of at least 1e-2 at
every layer, so that a few-ulp difference between the GPU's and the
oracle's bf16 hidden states cannot flip a selection.  Calls only oracle/
and the input generators.
"""
import json
import os
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import moe_inputs as G  # noqa: E402
import oracle as O  # noqa: E402

MIN_GAP = 1e-2


def oracle_layers(w):
    out = []
    for l in range(w.L):
        hx = G.HostExperts(w, l)
        out.append(dict(router=G.router_weights(w, l), gamma=G.gamma(w, l), k=w.k,
                        routed=hx.routed, shared=hx.shared()))
    return out


def main():
    w = G.WORKLOADS["k3_stack8"]
    layers = oracle_layers(w)
    pool = ThreadPoolExecutor(max_workers=os.cpu_count())
    for draw in range(64):
        h = G.token(w, draw)
        gaps = []
        ok = True
        for l, L in enumerate(layers):
            xn = O.rmsnorm_bf16(h, L["gamma"], w.eps)
            gap = float(O.topk_gap(O.router_logits(xn, L["router"]), w.k)[0])
            gaps.append(gap)
            if gap < MIN_GAP:
                ok = False
                break
            r = O.moe_layer(xn, L["router"], w.k, L["routed"], L["shared"], residual_bits=h,
                            pmap=pool.map)
            h = O.f64_to_bf16(r["out"])
        print(draw, ["%.4f" % g for g in gaps], flush=True)
        if ok:
            with open(os.path.join(HERE, "stack8_token.json"), "w") as f:
                json.dump({"workload": w.name, "draw": draw, "min_gap": MIN_GAP,
                           "layer_gaps": gaps}, f, indent=1)
            return
    raise SystemExit("no draw found")


if __name__ == "__main__":
    main()
