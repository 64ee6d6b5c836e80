"""The hand-worked two-token fixture of tests/golden/, embedded in d channels."""
import json
import os

import numpy as np

from gated_delta_rule_prefill_amd import inputs as gen

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "two_tokens_by_hand.json")


def load(d: int = 64, H: int = 1):
    """Inputs (fp32, [T=2, H, d]) with the example in channels 0..1 of every head,
    and the expected o [2, H, d] and final state [1, H, d, d] (zeros elsewhere)."""
    g = json.load(open(PATH))
    T = 2
    q = np.zeros((T, H, d), np.float32)
    k = np.zeros((T, H, d), np.float32)
    v = np.zeros((T, H, d), np.float32)
    la = np.zeros((T, H, d), np.float32)
    q[:, :, :2] = np.array(g["q"], np.float32)[:, None]
    k[:, :, :2] = np.array(g["k"], np.float32)[:, None]
    v[:, :, :2] = np.array(g["v"], np.float32)[:, None]
    la[:, :, :2] = np.log(np.array(g["alpha"], np.float64)).astype(np.float32)[:, None]
    beta = np.repeat(np.array(g["beta"], np.float32)[:, None], H, axis=1)
    o = np.zeros((T, H, d))
    o[:, :, :2] = np.array(g["o"])[:, None]
    fin = np.zeros((1, H, d, d))
    fin[0, :, :2, :2] = np.array(g["final_state"])[None]
    x = gen.KDAInputs(q=q, k=k, v=v, log_alpha=la, beta=beta, initial_state=None,
                      cu_seqlens=None, num_seqs=1, dtype="f32")
    return x, o, fin
