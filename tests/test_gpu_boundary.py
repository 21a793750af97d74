"""GPU tests of the boundary: the device input checks (DSPARK_CHECK_INPUTS,
dspark_check) and calls launched on a side stream.

The out-of-contract inputs used here are only those the kernels already
clamp into their buffers (token ids, uniforms, confidences, verify row
offsets that give a request no rows or too many): the checks must report
them, and every access stays in bounds whatever they hold.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_harness import Tally, compare_draft, compare_schedule, compare_verify, gpu_step, upload

pytestmark = pytest.mark.gpu


def _ds():
    import draft_verify_sampling_bias_amd as ds
    return ds


@pytest.mark.parametrize("R,wd", [(12, "bf16"), (80, "bf16"), (6, "f32")], ids=["seg16", "seg64", "seg32"])
def test_input_checks_clean_step(R, wd):
    """A whole step with the checks on and inputs inside the contract: no
    bit is set, and the results equal those of the unchecked step."""
    ds = _ds()
    inp = synth.make_custom(300 + R, R, 4, 3000, 64, wdtype=wd, policy="mixed", K_mode="uniformK")
    d = upload(inp)
    ref = gpu_step(d, inp.K, inp.gamma)
    y, q_tok, q_stats = ds.dspark_draft_block(d["U"], d["W1"], d["W2"], d["anchor"], d["temp"], d["u_draft"],
                                              check_inputs=True)
    sch = ds.dspark_schedule(d["c"], inp.K, d["anchor"], y, check_inputs=True)
    cut = ds.dspark_schedule_cutoff(d["c"], 0.5, d["anchor"], y, check_inputs=True)
    rows = d["target"][sch["row_req"].long(), sch["row_pos"].long()].contiguous()
    n_acc, out_tok, p_tok = ds.dspark_verify(rows, sch["row_offsets"], d["U"], d["W1"], d["W2"], d["anchor"],
                                             d["temp"], y, q_tok, q_stats, d["u_accept"], d["u_final"],
                                             check_inputs=True)
    torch.cuda.synchronize()
    got = dict(y=y, q_tok=q_tok, q_stats=q_stats, n_accept=n_acc, out_tok=out_tok, p_tok=p_tok, **sch)
    for k, v in got.items():
        if v is not None:
            np.testing.assert_array_equal(v.cpu().numpy(), ref[k], err_msg=k)
    assert int(cut["row_offsets"][-1]) >= R
    print(f"[checks clean {wd} R={R}] ok", flush=True)


def test_input_checks_report_bad_inputs():
    """Each kind of bad input sets its bit; a later call on the same
    workspace without the checks rewrites the word to 0."""
    ds = _ds()
    R, gamma, V, rank = 4, 3, 2000, 64
    inp = synth.make_custom(310, R, gamma, V, rank, policy="mixed")
    d = upload(inp)
    dev = d["U"].device
    ws_d = torch.empty(ds.draft_workspace_bytes(R, gamma, V, rank, ds.W_BF16, ds.CHECK_INPUTS), dtype=torch.uint8,
                       device=dev)

    def draft(anchor, u_draft, check=True):
        return ds.dspark_draft_block(d["U"], d["W1"], d["W2"], anchor, d["temp"], u_draft, workspace=ws_d,
                                     check_inputs=check)

    y, q_tok, q_stats = draft(d["anchor"], d["u_draft"])          # clean
    bad_anchor = d["anchor"].clone()
    bad_anchor[1] = V + 7
    bad_anchor[2] = -3
    with pytest.raises(ds.InputCheckError) as e:
        draft(bad_anchor, d["u_draft"])
    assert e.value.bits == ds.BAD_TOKEN
    bad_u = d["u_draft"].clone()
    bad_u[0, 1] = 1.0
    bad_u[3, 2] = float("nan")
    with pytest.raises(ds.InputCheckError) as e:
        draft(d["anchor"], bad_u)
    assert e.value.bits == ds.BAD_UNIFORM
    with pytest.raises(ds.InputCheckError) as e:
        draft(bad_anchor, bad_u)
    assert e.value.bits == ds.BAD_TOKEN | ds.BAD_UNIFORM
    # the word belongs to the last call: an unchecked call clears it
    draft(bad_anchor, bad_u, check=False)
    assert ds.dspark_check(ws_d) == 0

    # schedule: confidences outside [0, 1] or NaN, negative tokens
    bad_c = d["c"].clone()
    bad_c[0, 0] = 1.5
    bad_c[2, 1] = float("nan")
    with pytest.raises(ds.InputCheckError) as e:
        ds.dspark_schedule(bad_c, R * gamma, d["anchor"], y, check_inputs=True)
    assert e.value.bits == ds.BAD_CONFIDENCE
    with pytest.raises(ds.InputCheckError) as e:
        ds.dspark_schedule_cutoff(d["c"], 0.5, bad_anchor, y, check_inputs=True)
    assert e.value.bits == ds.BAD_TOKEN

    # verify: request 1 owns no row and request 2 owns gamma + 2 = 5 rows (the
    # rows stay inside [0, n_rows]); the verify kernels give those requests
    # n_accept 0 and out_tok -1 and leave the others as usual
    off = torch.tensor([0, 4, 4, 9, 12], dtype=torch.int32, device=dev)
    rows = torch.randn((12, V), device=dev)
    args = (rows, off, d["U"], d["W1"], d["W2"], d["anchor"], d["temp"], y, q_tok, q_stats)
    with pytest.raises(ds.InputCheckError) as e:
        ds.dspark_verify(*args, d["u_accept"], d["u_final"], check_inputs=True)
    assert e.value.bits == ds.BAD_LENGTH
    n_acc, out_tok, _ = ds.dspark_verify(*args, d["u_accept"], d["u_final"])
    assert int(out_tok[1]) == -1 and int(out_tok[2]) == -1 and int(n_acc[1]) == 0
    bad_ua = d["u_accept"].clone()
    bad_ua[1, 0] = 1.5
    bad_uf = d["u_final"].clone()
    bad_uf[3] = -0.25
    y_bad = y.clone()
    y_bad[0, 0] = V
    ok_off = torch.arange(R + 1, dtype=torch.int32, device=dev) * (gamma + 1)
    rows_ok = torch.randn((R * (gamma + 1), V), device=dev)
    with pytest.raises(ds.InputCheckError) as e:
        ds.dspark_verify(rows_ok, ok_off, d["U"], d["W1"], d["W2"], d["anchor"], d["temp"], y_bad, q_tok, q_stats,
                         bad_ua, bad_uf, check_inputs=True)
    assert e.value.bits == ds.BAD_TOKEN | ds.BAD_UNIFORM
    print("[checks bad inputs] every bit reported", flush=True)


@pytest.mark.parametrize("R", [20, 100])
def test_step_on_a_side_stream(R):
    """A step launched on a side stream, with every output and workspace
    allocated by the binding: while its kernels run, the current stream
    allocates and fills other tensors; the results equal those of the step on
    the current stream (the binding allocates from the side stream's pool,
    so no buffer of the step is handed out in between)."""
    ds = _ds()
    inp = synth.make_custom(320 + R, R, 5, 20000, 128, policy="temps", K_mode="uniformK")
    d = upload(inp)
    ref = gpu_step(d, inp.K, inp.gamma)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        y, q_tok, q_stats = ds.dspark_draft_block(d["U"], d["W1"], d["W2"], d["anchor"], d["temp"], d["u_draft"],
                                                  stream=side)
        sch = ds.dspark_schedule(d["c"], inp.K, d["anchor"], y, stream=side)
        with torch.cuda.stream(side):
            rows = d["target"][sch["row_req"].long(), sch["row_pos"].long()].contiguous()
        n_acc, out_tok, p_tok = ds.dspark_verify(rows, sch["row_offsets"], d["U"], d["W1"], d["W2"], d["anchor"],
                                                 d["temp"], y, q_tok, q_stats, d["u_accept"], d["u_final"],
                                                 stream=side)
        # churn on the current stream while the side stream works
        junk = [torch.full((1 << 20,), float(i), device="cuda") for i in range(8)]
        del junk
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        got = dict(y=y, q_tok=q_tok, q_stats=q_stats, n_accept=n_acc, out_tok=out_tok, p_tok=p_tok, **sch)
        for k, v in got.items():
            if v is not None:
                np.testing.assert_array_equal(v.cpu().numpy(), ref[k], err_msg=f"rep {rep} {k}")
    print(f"[side stream R={R}] identical", flush=True)
