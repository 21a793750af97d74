"""Host checks of the GPU parity harness's own arithmetic (no GPU)."""
import numpy as np

import gpu_harness as gh
import oracle
import synth


def test_own_q_of_flipped_tokens():
    """Where the GPU's drafted token differs from the oracle's own draw, the
    own-q re-verification must use the oracle's probability of the GPU's
    token (from the oracle's full logits of that position), and d.q_tok
    everywhere else."""
    inp = synth.make_custom(7, 4, 3, 50, 16, wdtype="bf16", policy="temps", K_mode="fixed", U_std=3.0,
                            noise_std=1.0)
    reqs = list(range(inp.R))
    d0 = oracle.draft_block(inp.U, inp.W1, inp.W2, inp.wdtype, inp.anchor, inp.temp, inp.u_draft)
    y_fake = d0.y.copy()
    flips = [(1, 0), (2, 2)]
    for r, k in flips:
        y_fake[r, k] = (int(d0.y[r, k]) + 7) % inp.V
    d = oracle.draft_block(inp.U, inp.W1, inp.W2, inp.wdtype, inp.anchor, inp.temp, inp.u_draft,
                           prev_override=y_fake, keep_s=True)
    q = gh.own_q_of_gpu_tokens(inp, {"y": y_fake}, d, reqs)
    for r in reqs:
        for k in range(inp.gamma):
            if (r, k) in flips:
                x = d.s[(r, k)] / oracle._sample_T(float(inp.temp[r]))
                w = np.exp(x - x.max())
                want = w[y_fake[r, k]] / w.sum()
                assert y_fake[r, k] != d.y[r, k]
                assert abs(q[r, k] - want) <= 1e-12 * want, (r, k, q[r, k], want)
                assert abs(q[r, k] - d.q_tok[r, k]) > 1e-6 * want  # a different token's probability
            else:
                assert q[r, k] == d.q_tok[r, k]
