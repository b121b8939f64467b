"""Write the stored expected values under tests/golden/.

Calls only ``oracle/`` and the seeded input generators: no value here comes
from the HIP library.  Run from the repo root:  python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from combine_get_dispatch_histogram_amd import workloads as wl  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def tiny():
    w = wl.TINY
    inp = wl.normal_inputs(w, 0)
    idx = inp["topk_idx"].numpy()
    x = wl.bf16_bits(inp["x"])
    wts = inp["topk_weights"].numpy()
    lay = oracle.layout(idx, w.S, w.E, w.R)
    d = oracle.dispatch(x, idx, wts, lay["is_token_in_rank"], lay["num_tokens_per_expert"], S=w.S, E=w.E, R=w.R,
                        C=w.C)
    c = oracle.combine(d["recv_x"], d["recv_topk_weights"], d["send_head"], d["recv_rank_offset"], S=w.S)
    codes, sci, ue = oracle.fp8_quantize(x, True)
    return {
        "workload": "tiny: 4 sources x 32 tokens, hidden 256, 16 experts on 4 ranks, top-4, 24 channels, seed 0",
        "inputs_sha256": {"x": sha(x), "topk_idx": sha(idx), "topk_weights": sha(wts)},
        "num_tokens_per_rank": lay["num_tokens_per_rank"].tolist(),
        "num_tokens_per_expert": lay["num_tokens_per_expert"].tolist(),
        "is_token_in_rank_sha256": sha(lay["is_token_in_rank"]),
        "rank_prefix_matrix": d["rank_prefix_matrix"].tolist(),
        "recv_rank_offset": d["recv_rank_offset"].tolist(),
        "channel_prefix_matrix_sha256": sha(d["channel_prefix_matrix"]),
        "recv_channel_prefix_matrix_sha256": sha(d["recv_channel_prefix_matrix"]),
        "send_head_sha256": sha(d["send_head"]),
        "recv_src_idx_sha256": sha(d["recv_src_idx"]),
        "recv_x_sha256": sha(d["recv_x"]),
        "recv_topk_idx_sha256": sha(d["recv_topk_idx"]),
        "recv_topk_weights_sha256": sha(d["recv_topk_weights"]),
        "num_recv_tokens_per_expert": d["num_recv_tokens_per_expert"].tolist(),
        "combined_x_sha256": sha(c["combined_x"]),
        "combined_topk_weights_sha256": sha(c["combined_topk_weights"]),
        "fp8_round_scale_codes_sha256": sha(codes),
        "fp8_round_scale_scales_sha256": sha(sci),
    }


if __name__ == "__main__":
    oracle.build()
    with open(os.path.join(HERE, "tiny_seed0.json"), "w") as f:
        json.dump(tiny(), f, indent=1)
        f.write("\n")
    print("wrote", os.path.join(HERE, "tiny_seed0.json"))
