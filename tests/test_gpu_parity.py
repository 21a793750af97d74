"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small cases are compared in full.  The full-size configurations are compared
exactly on the schedule; draft and verify are compared on every request at
R <= 64 and, above that, on 64 requests spread evenly over the batch (one per
stratum of R / 64 consecutive requests, so every 16-request chunk window and
every 256-request window of the large-batch kernels is visited).  Every
request's draft and verify are independent of the others.
"""
import numpy as np
import pytest
import torch  # noqa: F401  (first import is slow on a fresh box: pay it at collection)

import synth
from gpu_harness import Tally, compare_draft, compare_schedule, compare_verify, gpu_step, upload, upload_A

pytestmark = pytest.mark.gpu


def _run(inp, K=None, reqs=None, label=""):
    K = inp.K if K is None else K
    d = upload(inp)
    g = gpu_step(d, K, inp.gamma)
    reqs = list(range(inp.R)) if reqs is None else list(reqs)
    t = Tally()
    dr = compare_draft(inp, g, reqs, t)
    compare_schedule(inp, g, K)
    compare_verify(inp, g, reqs, t, dr)
    print(f"[{label or inp.name}] K={K} {t.summary()}", flush=True)
    t.check()
    return g


@pytest.mark.parametrize("policy", ["greedy", "sampled"])
def test_config1(policy):
    _run(synth.make_config(1, policy))


SMALL = [
    # (seed, R, gamma, V, rank, wdtype, policy, K_mode)
    (11, 3, 4, 1000, 64, "bf16", "sampled", "fixed"),        # ragged last tile, one chunk
    (12, 3, 4, 1000, 64, "bf16", "greedy", "fixed"),
    (13, 70, 3, 4099, 40, "bf16", "temps", "uniformK"),      # V % 4 != 0, rank % 16 == 8, 2 chunks
    (14, 130, 2, 2300, 512, "bf16", "mixed", "uniformK"),    # 3 request chunks, rank 512
    (15, 5, 3, 777, 24, "f32", "temps", "fixed"),            # fp32 weights
    (16, 33, 6, 1536, 256, "f32", "mixed", "uniformK"),      # fp32, 2 chunks
    (17, 2, 1, 9000, 8, "bf16", "sampled", "fixed"),         # gamma = 1, minimum rank
    (18, 9, 16, 513, 128, "bf16", "temps", "uniformK"),      # maximum gamma
    (19, 4, 5, 5, 16, "bf16", "sampled", "fixed"),           # tiny vocabulary
    (20, 3, 2, 300000, 64, "bf16", "mixed", "fixed"),        # > 16384 segment records: unstaged finish
    (21, 2, 2, 600000, 8, "f32", "temps", "fixed"),          # same on the 32-row path, 147 chunks
    # 64-row path (bf16, R > 64): request chunks of 16, info windows of 256
    (25, 300, 3, 3001, 128, "bf16", "mixed", "uniformK"),    # 19 chunks (odd), 2 windows, V % 4 != 0
    (26, 600, 2, 4160, 256, "bf16", "temps", "fixed"),       # 38 chunks, 3 windows, ragged last window
    (27, 65, 3, 5000, 512, "bf16", "sampled", "uniformK"),   # one request in the last chunk
    (28, 97, 2, 1000, 96, "bf16", "sampled", "fixed"),       # rank 96: zero k-groups in the last step
    # ranks whose next-to-last k-step is not full: k-groups past the rank
    # before the last k-step
    (29, 70, 3, 1000, 24, "bf16", "mixed", "uniformK"),      # rank 24: one such group in the first step
    (30, 80, 2, 777, 8, "bf16", "sampled", "fixed"),         # rank 8: one real k-group
    (31, 66, 2, 2000, 72, "bf16", "temps", "fixed"),         # rank 72: 4 k-steps, the third partial
    (32, 90, 2, 1500, 200, "bf16", "mixed", "uniformK"),     # rank 200: 8 k-steps, the seventh partial
    (33, 67, 2, 1200, 384, "bf16", "sampled", "fixed"),      # rank 384: 16 k-steps, the last four empty
    (34, 40, 3, 3000, 200, "bf16", "mixed", "uniformK"),     # the same ranks on the 16-row path
    (35, 64, 2, 2000, 384, "bf16", "sampled", "fixed"),
    (36, 10, 2, 1000, 200, "f32", "temps", "fixed"),         # and on the fp32 path
    (37, 70, 3, 5, 16, "bf16", "mixed", "uniformK"),         # tiny vocabularies on the 64-row path
    (38, 66, 2, 4, 8, "bf16", "sampled", "fixed"),           # (one segment, V % 4 == 0)
    (39, 3, 2, 4, 8, "f32", "sampled", "fixed"),             # and on the fp32 path
    (40, 2, 2, 200000, 16, "bf16", "mixed", "fixed"),        # 12500 records: staged in two batches
    (41, 3, 2, 32768, 64, "bf16", "sampled", "fixed"),       # 2048 records: the small stage, full
    (42, 3, 2, 32784, 64, "bf16", "sampled", "fixed"),       # 2049 records: the large stage
    (43, 70, 16, 1000, 64, "bf16", "temps", "uniformK"),     # maximum gamma on the 64-row path
    (44, 33, 16, 1000, 96, "f32", "mixed", "uniformK"),      # and on the fp32 path
    # the wave-range draft finish (1024 threads: 4, 8 or 12 records per lane,
    # 256 threads above 256 requests) at the edges of each size
    (50, 2, 2, 65536, 16, "bf16", "sampled", "fixed"),       # 4096 records: 4 per lane, full
    (51, 2, 2, 65552, 16, "bf16", "mixed", "fixed"),         # 4097: 8 per lane
    (52, 3, 2, 131088, 16, "bf16", "temps", "fixed"),        # 8193: 12 per lane
    (53, 2, 2, 196608, 8, "bf16", "sampled", "fixed"),       # 12288: 12 per lane, full
    (54, 2, 2, 196624, 8, "bf16", "sampled", "fixed"),       # 12289: the staged finish
    (55, 70, 2, 262208, 8, "bf16", "mixed", "fixed"),        # 64-row segments, 4097 records: 8 per lane
    (56, 260, 2, 65600, 8, "bf16", "sampled", "fixed"),      # 256 threads, 1025 records: 8 per lane
    # many request windows on the 64-row path (each window: 256 requests,
    # loaded one window ahead into the other LDS half)
    (57, 2990, 2, 1000, 32, "bf16", "mixed", "uniformK"),    # 187 chunks (odd), 12 windows, ragged last
    (58, 5000, 3, 600, 64, "bf16", "temps", "uniformK"),     # 313 chunks, 20 windows
]


@pytest.mark.parametrize("case", SMALL, ids=[f"s{c[0]}" for c in SMALL])
def test_small_shapes(case):
    seed, R, gamma, V, rank, wd, pol, km = case
    inp = synth.make_custom(seed, R, gamma, V, rank, wdtype=wd, policy=pol, K_mode=km, U_std=3.0, noise_std=1.0)
    _run(inp)


def random_shapes(n, seed):
    """n seeded random step shapes inside the library's limits, over every
    path (16-row and 64-row bf16, fp32 weights), every policy and capacity
    mode, Zipf-shaped or normal base logits, sized so that the oracle takes
    about a second for each."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        wd = "f32" if rng.random() < 0.2 else "bf16"
        wide = wd == "bf16" and rng.random() < 0.5
        R = (int(rng.choice([65, 66, 79, 80, 95, 96, 97, 128, 129, 255, 256, 257, 300, 511, 513, 700, 1024, 1100]))
             if wide else int(rng.integers(1, 65)))
        gamma = int(rng.integers(1, 17))
        rank = int(8 * rng.integers(1, 65))
        V = int(rng.choice([int(rng.integers(2, 200)), int(rng.integers(200, 5000)), int(rng.integers(5000, 70000))]))
        pol = str(rng.choice(["greedy", "sampled", "temps", "mixed"]))
        km = str(rng.choice(["fixed", "uniformK", "2R"]))
        seed_i = int(rng.integers(1, 1 << 30))
        zipf = float(rng.choice([0.0, 1.1])) or None
        noise = float(rng.choice([0.5, 1.0]))
        if R * gamma * V * rank > 2.5e10 or R * V > 4e7 or (R + 1023) // 1024 * gamma > 16:
            continue
        if km == "uniformK" and gamma < 2:  # K ~ U{R .. R gamma / 2} needs gamma >= 2
            km = "fixed"
        out.append((seed_i, R, gamma, V, rank, wd, pol, km, zipf, noise))
    return out


# a flagged CDF-boundary flip at a draft position, where the re-verification
# must take the oracle's q of the GPU's token
RANDOM = [(648926920, 256, 3, 29075, 224, "bf16", "mixed", "uniformK", None, 1.0)] + random_shapes(40, 20240)


@pytest.mark.parametrize("case", RANDOM, ids=[f"rnd{i}" for i in range(len(RANDOM))])
def test_random_shapes(case):
    seed, R, gamma, V, rank, wd, pol, km, zipf, noise = case
    name = f"random seed={seed} R={R} gamma={gamma} V={V} rank={rank} {wd} {pol} {km} zipf={zipf} noise={noise}"
    print(name, flush=True)
    inp = synth.make_custom(seed, R, gamma, V, rank, wdtype=wd, policy=pol, K_mode=km, zipf=zipf,
                            U_std=None if zipf else 3.0, noise_std=noise, name=name)
    _run(inp)


@pytest.mark.parametrize("case", random_shapes(12, 4242), ids=[f"rndp{i}" for i in range(12)])
def test_random_shapes_packed_or_cutoff(case):
    """Random shapes again, half with the fragment-packed W2 and the top-K
    schedule (bf16, R <= 64: the layout of the 16-row kernel), the rest with
    the static cutoff schedule at a random confidence threshold."""
    seed, R, gamma, V, rank, wd, pol, km, zipf, noise = case
    use_pack = wd == "bf16" and R <= 64 and seed % 2 == 0
    conf_min = (0.05, 0.3, 0.6, 0.9)[seed % 4]
    name = f"random seed={seed} R={R} gamma={gamma} V={V} rank={rank} {wd} {pol} {km} zipf={zipf} noise={noise}"
    name += " packed" if use_pack else f" cutoff {conf_min}"
    print(name, flush=True)
    inp = synth.make_custom(seed, R, gamma, V, rank, wdtype=wd, policy=pol, K_mode=km, zipf=zipf,
                            U_std=None if zipf else 3.0, noise_std=noise, name=name)
    d = upload(inp)
    reqs = list(range(R))
    t = Tally()
    if use_pack:
        import draft_verify_sampling_bias_amd as ds
        g = gpu_step(d, inp.K, gamma, W2_packed=ds.dspark_pack_w2(d["W2"]))
        dr = compare_draft(inp, g, reqs, t)
        compare_schedule(inp, g, inp.K)
    else:
        g = gpu_step(d, None, gamma, conf_min=conf_min)
        dr = compare_draft(inp, g, reqs, t)
        compare_schedule(inp, g, None, conf_min=conf_min)
    compare_verify(inp, g, reqs, t, dr)
    print(f"[{name}] {t.summary()}", flush=True)
    t.check()


def masked_extreme(seed, R, gamma, V, rank, wd, pol, km, dens, n_ext):
    """Inputs of a random shape with a -inf mask of density dens drawn per
    (request, position) row of U (one entry of each row kept finite) and at
    half that density per target row, and n_ext requests at extreme
    temperatures (+inf, 1e35, 1e30, subnormal, 1e-30, 1e-3, NaN, negative,
    50, 1, 0)."""
    ext = np.array([np.inf, 1e35, 1e30, 1e-40, 1e-30, 1e-3, np.nan, -1.0, 50.0, 1.0, 0.0], np.float32)
    inp = synth.make_custom(seed, R, gamma, V, rank, wdtype=wd, policy=pol, K_mode=km, U_std=3.0, noise_std=1.0,
                            name=f"masked seed={seed} R={R} gamma={gamma} V={V} rank={rank} {wd} dens={dens}")
    rng = np.random.default_rng(seed)
    m = rng.random(inp.U.shape) < dens
    keep = rng.integers(0, V, size=inp.U.shape[:2])
    m[np.arange(R)[:, None], np.arange(gamma)[None, :], keep] = False
    inp.U[m] = -np.inf
    mt = rng.random(inp.target.shape) < dens * 0.5
    kt = rng.integers(0, V, size=inp.target.shape[:2])
    mt[np.arange(R)[:, None], np.arange(gamma + 1)[None, :], kt] = False
    inp.target[mt] = -np.inf
    if n_ext:
        idx = rng.choice(R, size=min(R, n_ext), replace=False)
        inp.temp[idx] = ext[rng.integers(0, len(ext), size=idx.size)]
    return inp


MASKED = [
    # fp32 weights, one finite entry per row, T = 1e-40: the rescan's logits
    # differ from the records' by rounding, which c ~ 1.4e30 magnified
    (442002694, 48, 8, 13, 488, "f32", "temps", "2R", 0.99, 3),
    # the same on the 64-row bf16 path
    (671932773, 300, 10, 131, 184, "bf16", "temps", "fixed", 0.9, 3),
    # T = 1e-3 with a second entry 0.0025 below the maximum: q and Z within
    # the fp32 logits' rounding magnified by 1 / T
    (864547394, 60, 5, 22824, 80, "bf16", "mixed", "2R", 0.5, 2),
    (313279300, 256, 5, 24, 328, "bf16", "mixed", "fixed", 0.5, 3),
    (417947361, 6, 7, 19113, 120, "bf16", "mixed", "uniformK", 0.99, 2),
    (512710369, 47, 5, 15408, 224, "bf16", "temps", "2R", 0.5, 0),
]


@pytest.mark.parametrize("case", MASKED, ids=[f"mask{i}" for i in range(len(MASKED))])
def test_random_masks_and_extreme_temperatures(case):
    print("masked", case, flush=True)
    _run(masked_extreme(*case))


def test_target_only_fallback_K0():
    """K = 0: nothing is verified, one row per request, the emitted token is
    the bonus draw from row 0 (target-only decoding)."""
    inp = synth.make_custom(21, 16, 4, 3000, 64, policy="mixed")
    g = _run(inp, K=0)
    assert (g["l"] == 0).all() and (g["n_accept"] == 0).all()


@pytest.mark.parametrize("R,wd", [(10, "bf16"), (70, "bf16"), (10, "f32")], ids=["seg16", "seg64", "seg32"])
def test_extreme_temperatures(R, wd):
    """Temperatures at and past the ends of the clamp [1e-30, 1e30]: +inf and
    1e35 sample uniformly over the entries that are not -inf, a subnormal and
    1e-30 sample the argmax, NaN and a negative value are greedy; some
    entries are masked (-inf) in U and in the target."""
    inp = synth.make_custom(60 + R, R, 3, 3000, 64, wdtype=wd, policy="temps", K_mode="fixed", U_std=3.0,
                            noise_std=1.0)
    extremes = np.array([np.inf, 1e35, 1e30, 1e-40, 1e-30, 1e-3, np.nan, -1.0, 50.0, 1.0], np.float32)
    inp.temp[:] = extremes[np.arange(R) % len(extremes)]
    rng = np.random.default_rng(90 + R)
    mask = rng.random(inp.V) < 0.3
    inp.U[:, :, mask] = -np.inf
    inp.target[:, :, mask | (rng.random(inp.V) < 0.1)] = -np.inf
    _run(inp, label=f"extreme-T-{wd}-R{R}")


def test_high_acceptance_and_greedy_identity():
    """Target = drafter base logits with small noise and no Markov bias: most
    drafts are accepted; greedy requests emit the target argmax chain."""
    inp = synth.make_custom(22, 24, 5, 2048, 32, policy="mixed", noise_std=0.05, W_std=0.0)
    g = _run(inp)
    assert g["n_accept"].mean() > 1.0
    rows, off = g["rows"], g["row_offsets"]
    for r in np.flatnonzero(inp.temp <= 0):
        n = g["n_accept"][r]
        am = [int(np.argmax(rows[off[r] + j])) for j in range(n + 1)]
        assert list(g["y"][r, :n]) + [int(g["out_tok"][r])] == am


def test_run_twice_bit_identical():
    import draft_verify_sampling_bias_amd  # noqa: F401
    inp = synth.make_custom(23, 40, 5, 5000, 256, policy="mixed", K_mode="uniformK")
    d = upload(inp)
    g1 = gpu_step(d, inp.K, inp.gamma)
    g2 = gpu_step(d, inp.K, inp.gamma)
    for k in g1:
        np.testing.assert_array_equal(g1[k], g2[k], err_msg=k)


@pytest.mark.parametrize("R,wd", [(20, "bf16"), (70, "bf16"), (40, "f32")], ids=["seg16", "seg64", "seg32"])
def test_masked_vocabulary(R, wd):
    """Logits of -inf (a vocabulary mask): whole 16/32/64-row segments and a
    whole 4096-entry target chunk masked, plus scattered entries; the target
    masks some entries the drafter allows, so p = 0 for some drafted tokens."""
    inp = synth.make_custom(24 + R, R, 4, 9000, 64, wdtype=wd, policy="mixed", K_mode="uniformK", U_std=3.0,
                            noise_std=1.0)
    rng = np.random.default_rng(2024 + R)
    mask = np.zeros(inp.V, bool)
    mask[1000:1600] = True
    mask[8192:] = True
    mask |= rng.random(inp.V) < 0.2
    inp.U[:, :, mask] = -np.inf
    inp.target[:, :, mask | (rng.random(inp.V) < 0.1)] = -np.inf
    g = _run(inp, label=f"masked-R{R}")
    assert not np.isin(g["y"], np.flatnonzero(mask)).any()


@pytest.mark.parametrize("R,gamma", [(1, 1), (37, 5), (64, 7), (1500, 3), (5000, 3)])
def test_schedule_cutoff(R, gamma):
    """Static confidence cutoff against the oracle, bit-exact, with exact ties
    at conf_min, NaN and out-of-range confidences, and several 1024-request
    rounds per thread."""
    import torch
    import draft_verify_sampling_bias_amd as ds
    import oracle
    rng = np.random.default_rng(700 + R + gamma)
    c = (1 / (1 + np.exp(-rng.normal(1, 1, (R, gamma))))).astype(np.float32)
    c.flat[::7] = np.float32(0.5)
    c.flat[::23] = np.float32(0.3)
    c.flat[3::29] = np.nan
    c.flat[5::31] = np.float32(1.25)
    c.flat[6::37] = np.float32(-0.5)
    anc = rng.integers(0, 100000, R).astype(np.int32)
    y = rng.integers(0, 100000, (R, gamma)).astype(np.int32)
    cd, ad, yd = (torch.from_numpy(x).cuda() for x in (c, anc, y))
    for conf_min in (-1.0, 0.0, 0.3, 0.5, 0.6, 0.999, 1.0, 1.5):
        g = {k: v.cpu().numpy() for k, v in ds.dspark_schedule_cutoff(cd, conf_min, ad, yd).items()}
        o = oracle.schedule_cutoff(c, conf_min, anc, y)
        n = int(o.row_offsets[-1])
        np.testing.assert_array_equal(g["a"], o.a)
        np.testing.assert_array_equal(g["l"], o.l, err_msg=f"conf_min={conf_min}")
        np.testing.assert_array_equal(g["row_offsets"], o.row_offsets)
        for f in ("row_req", "row_pos", "row_tok"):
            np.testing.assert_array_equal(g[f][:n], getattr(o, f), err_msg=f)
        assert abs(float(g["expected_tokens"][0]) - o.expected_tokens) <= 1e-5 * o.expected_tokens
    print(f"[cutoff R={R} gamma={gamma}] ok", flush=True)


@pytest.mark.parametrize("cfg,conf_min", [(3, 0.6), (4, 0.3)])
def test_cutoff_step(cfg, conf_min):
    """A full step with the static cutoff in place of the top-K scheduler:
    draft, cutoff schedule, verify on the variable-length rows (sampled
    requests compared against the oracle)."""
    inp = synth.make_config(cfg)
    reqs = _spread(inp.R, 64, cfg)
    d = upload(inp)
    g = gpu_step(d, None, inp.gamma, conf_min=conf_min)
    t = Tally()
    dr = compare_draft(inp, g, reqs, t)
    compare_schedule(inp, g, None, conf_min=conf_min)
    compare_verify(inp, g, reqs, t, dr)
    print(f"[cutoff config{cfg} conf_min={conf_min}] rows={int(g['row_offsets'][-1])} {t.summary()}", flush=True)
    t.check()


def _pack_reference(W2_bits, rank):
    """The fragment-packed layout built with NumPy from its definition in
    include/dspark.h (bf16 bit patterns)."""
    V = W2_bits.shape[0]
    KS = 2 if rank <= 64 else 4 if rank <= 128 else 8 if rank <= 256 else 16
    n_seg = (V + 15) // 16
    full = np.zeros((n_seg * 16, KS * 32), dtype=np.uint16)
    full[:V, :rank] = W2_bits
    # [s, i, ks, q, e] -> [s, ks, q, i, e]: slot L = 16 q + i of (s, ks)
    return full.reshape(n_seg, 16, KS, 4, 8).transpose(0, 2, 3, 1, 4).reshape(-1)


@pytest.mark.parametrize("V,rank", [(37, 8), (1000, 96), (4160, 512), (513, 128), (5, 16)])
def test_pack_w2_layout(V, rank):
    import torch
    import draft_verify_sampling_bias_amd as ds
    rng = np.random.default_rng(V + rank)
    bits = rng.integers(0, 1 << 16, (V, rank), dtype=np.uint16)
    W2 = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    got = ds.dspark_pack_w2(W2).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, _pack_reference(bits, rank))


@pytest.mark.parametrize("case", [(11, 3, 4, 1000, 64, "sampled"), (13, 40, 3, 4099, 40, "temps"),
                                  (18, 9, 16, 513, 128, "temps"), (19, 4, 5, 5, 16, "sampled"),
                                  (29, 64, 2, 20000, 512, "mixed"), (34, 40, 3, 3000, 200, "mixed"),
                                  (35, 20, 2, 2000, 384, "sampled")],
                         ids=["p11", "p13", "p18", "p19", "p29", "p34", "p35"])
def test_packed_w2_identical(case):
    """The fragment-packed W2 gives bit-identical results to W2 itself (the
    same products in the same order), and those match the oracle."""
    import draft_verify_sampling_bias_amd as ds
    seed, R, gamma, V, rank, pol = case
    inp = synth.make_custom(seed, R, gamma, V, rank, policy=pol, K_mode="uniformK", U_std=3.0, noise_std=1.0)
    d = upload(inp)
    g0 = gpu_step(d, inp.K, inp.gamma)
    g1 = gpu_step(d, inp.K, inp.gamma, W2_packed=ds.dspark_pack_w2(d["W2"]))
    for k in g0:
        np.testing.assert_array_equal(g1[k], g0[k], err_msg=k)
    t = Tally()
    dr = compare_draft(inp, g1, range(R), t)
    compare_verify(inp, g1, range(R), t, dr)
    print(f"[packed {inp.name}] {t.summary()}", flush=True)
    t.check()


def test_packed_w2_config3():
    import draft_verify_sampling_bias_amd as ds
    inp = synth.make_config(3)
    d = upload(inp)
    g0 = gpu_step(d, inp.K, inp.gamma)
    g1 = gpu_step(d, inp.K, inp.gamma, W2_packed=ds.dspark_pack_w2(d["W2"]))
    for k in g0:
        np.testing.assert_array_equal(g1[k], g0[k], err_msg=k)
    print("[packed config3] identical", flush=True)


def _spread(R, n, seed):
    """Every request when R <= n; otherwise one seeded request from each of
    n equal strata of consecutive requests (so the whole batch is visited)."""
    if R <= n:
        return list(range(R))
    rng = np.random.default_rng(seed)
    edges = [(i * R) // n for i in range(n + 1)]
    return [int(rng.integers(edges[i], edges[i + 1])) for i in range(n)]


@pytest.mark.parametrize("cfg,policy", [(2, "greedy"), (2, "sampled"), (3, None), (4, None), (5, None)])
def test_full_size_configs(cfg, policy):
    inp = synth.make_config(cfg, policy)
    reqs = _spread(inp.R, 64, cfg)
    if cfg == 5:
        assert (inp.temp[reqs] <= 0).any() and (inp.temp[reqs] > 0).any()
        assert len({r // 256 for r in reqs}) == 4
    _run(inp, reqs=reqs, label=f"config{cfg}-{policy or 'default'}")


def _capacity_case(rng, R, gamma, kind):
    c = (1 / (1 + np.exp(-rng.normal(1, 1, (R, gamma))))).astype(np.float32)
    import oracle
    a = oracle.survival(c) if R > 0 else np.zeros((0, gamma), np.float32)
    if kind == "raw" and a.size:
        # unsorted values with the clamping cases: NaN, negatives, -0, > 1,
        # subnormals and exact duplicates
        a = rng.random((R, gamma)).astype(np.float32)
        a.flat[::11] = np.nan
        a.flat[1::13] = np.float32(-0.25)
        a.flat[2::17] = np.float32(-0.0)
        a.flat[3::19] = np.float32(3.0)
        a.flat[4::23] = np.float32(1e-40)
        a.flat[5::7] = np.float32(0.5)
    return a


def _capacity_tables(rng, R, gamma):
    n_full = R * (gamma + 1) + 1
    yield "bucketed", synth.sps_table(n_full)
    yield "bucketed-steep", synth.sps_table(n_full, t_row=1.0 / 1024)
    yield "random-steps", synth.random_sps_table(int(rng.integers(1 << 30)), n_full)
    yield "per-row", np.array([1.0 / max(b, 1) for b in range(n_full)], np.float32)
    yield "constant", np.full(n_full, 3.0, np.float32)
    yield "short", synth.sps_table(R + 1 + int(rng.integers(0, max(1, R * gamma // 2))))
    yield "minimal", np.full(R + 1, 2.0, np.float32)
    nan_t = synth.sps_table(n_full)
    nan_t[R + (R * gamma) // 3] = np.nan
    yield "with-nan", nan_t


@pytest.mark.parametrize("R,gamma,kind", [(0, 3, "surv"), (1, 1, "surv"), (3, 5, "raw"), (64, 7, "surv"),
                                          (64, 7, "raw"), (256, 5, "surv"), (1000, 3, "raw"),
                                          (1024, 5, "surv")])
def test_capacity(R, gamma, kind):
    """Hardware-aware capacity against the oracle: K exact, E(K) and
    Theta(K) bit-identical (both round the exact sum once to fp64), over
    step-shaped, per-row, constant, short, minimal and NaN-holding tables."""
    import torch
    import draft_verify_sampling_bias_amd as ds
    import oracle
    rng = np.random.default_rng(900 + 7 * R + gamma)
    a = _capacity_case(rng, R, gamma, kind)
    ad = torch.from_numpy(a).cuda()
    for name, sps in _capacity_tables(rng, R, gamma):
        g = {k: v.cpu().numpy() for k, v in ds.dspark_capacity(ad, torch.from_numpy(sps).cuda()).items()}
        o = oracle.capacity(a, sps)
        assert int(g["K"][0]) == o.K, (name, int(g["K"][0]), o.K)
        assert float(g["expected"][0]) == o.expected, (name, float(g["expected"][0]), o.expected)
        th = float(g["theta"][0])
        assert th == o.theta or (np.isnan(th) and np.isnan(o.theta)), (name, th, o.theta)
        print(f"[capacity R={R} gamma={gamma} {kind} {name}] K={o.K} E={o.expected:.6f}", flush=True)


def test_capacity_largest_batch():
    """R * gamma = 16384 candidates (the limit): a constant rate takes every
    positive value, a bucketed rate stops inside the batch."""
    import torch
    import draft_verify_sampling_bias_amd as ds
    import oracle
    rng = np.random.default_rng(990)
    R, gamma = 1024, 16
    a = _capacity_case(rng, R, gamma, "surv")
    a.flat[::9] = np.float32(0.0)
    ad = torch.from_numpy(a).cuda()
    for sps in (np.full(R * (gamma + 1) + 1, 5.0, np.float32), synth.sps_table(R * (gamma + 1) + 1, t_row=1 / 65536)):
        g = {k: v.cpu().numpy() for k, v in ds.dspark_capacity(ad, torch.from_numpy(sps).cuda()).items()}
        o = oracle.capacity(a, sps)
        assert int(g["K"][0]) == o.K
        assert float(g["expected"][0]) == o.expected and float(g["theta"][0]) == o.theta
        print(f"[capacity R={R} gamma={gamma}] K={o.K}", flush=True)


@pytest.mark.parametrize("cfg", [3, 4])
def test_capacity_drives_the_schedule(cfg):
    """The lagged pipeline on the GPU: survival from dspark_schedule, capacity
    from that survival, then a schedule with that capacity; every result
    against the oracle."""
    import torch
    import draft_verify_sampling_bias_amd as ds
    import oracle
    inp = synth.make_config(cfg)
    c = torch.from_numpy(inp.c).cuda()
    anc = torch.from_numpy(inp.anchor).cuda()
    y = torch.from_numpy(inp.anchor[:, None].repeat(inp.gamma, 1)).cuda()
    s0 = ds.dspark_schedule(c, inp.R * inp.gamma, anc, y)
    sps = synth.sps_table(inp.R * (inp.gamma + 1) + 1)
    cap = ds.dspark_capacity(s0["a"], torch.from_numpy(sps).cuda())
    K = int(cap["K"].cpu()[0])
    o = oracle.capacity(oracle.survival(inp.c), sps)
    assert K == o.K and float(cap["expected"].cpu()[0]) == o.expected
    s1 = {k: v.cpu().numpy() for k, v in ds.dspark_schedule(c, K, anc, y).items()}
    os_ = oracle.schedule(inp.c, K, inp.anchor, y.cpu().numpy())
    np.testing.assert_array_equal(s1["l"], os_.l)
    np.testing.assert_array_equal(s1["row_offsets"], os_.row_offsets)
    assert abs(float(s1["expected_tokens"][0]) - o.expected) <= 1e-5 * o.expected
    print(f"[capacity config{cfg}] K={K} rows={int(s1['row_offsets'][-1])} E={o.expected:.3f}", flush=True)


@pytest.mark.parametrize("N,gamma,kind", [(1, 1, "model"), (37, 5, "model"), (2000, 7, "model"),
                                          (8192, 5, "model"), (8193, 5, "model"), (40000, 16, "model"),
                                          (3000, 4, "special"), (0, 3, "model")])
def test_sts_fit(N, gamma, kind):
    """Sequential temperature scaling fit against the oracle (tau within
    1e-6 relative: both solve the same score equation to fp64 precision,
    the GPU returns fp32), on both the register (N <= 8192) and streaming
    paths, with the degenerate positions (unreached, all-zero logits,
    separable) and clamped logits."""
    import torch
    import draft_verify_sampling_bias_amd as ds
    import oracle
    z, n_acc, _ = synth.make_calibration(800 + N + gamma, N, gamma)
    if kind == "special":
        z[:, 0] = np.float32(0.0)                        # no information at position 0
        z[:, 1] = np.where(n_acc > 1, 2.0, -2.0)         # separable at position 1
        z[::5, 2] = np.nan                               # NaN -> 0
        z[1::7, 3] = np.float32(1e30)                    # clamped
        n_acc = np.minimum(n_acc, 3).astype(np.int32)    # position 3 reached, never passed
    zd, nd = torch.from_numpy(z).cuda(), torch.from_numpy(n_acc).cuda()
    tau = ds.dspark_sts_fit(zd, nd).cpu().numpy()
    o = oracle.sts_fit(z, n_acc)
    np.testing.assert_allclose(tau, o.tau.astype(np.float32), rtol=1e-6, err_msg=f"{o.tau}")
    print(f"[sts fit N={N} gamma={gamma} {kind}] tau={np.round(tau, 4).tolist()}", flush=True)


@pytest.mark.parametrize("R,gamma", [(1, 1), (64, 7), (1000, 16), (5000, 3)])
def test_sts_apply_and_schedule(R, gamma):
    """Calibrated confidence against the oracle, then the schedule on it."""
    import torch
    import draft_verify_sampling_bias_amd as ds
    import oracle
    rng = np.random.default_rng(850 + R)
    z = rng.normal(1.5, 2.5, (R, gamma)).astype(np.float32)
    z.flat[::13] = np.nan
    z.flat[1::17] = np.float32(-300.0)
    z.flat[2::19] = np.float32(300.0)
    tau = rng.uniform(0.3, 3.0, gamma).astype(np.float32)
    c = ds.dspark_sts_apply(torch.from_numpy(z).cuda(), torch.from_numpy(tau).cuda())
    o = oracle.sts_apply(z, tau)
    g = c.cpu().numpy()
    tiny = np.finfo(np.float32).tiny
    big = o >= tiny
    np.testing.assert_allclose(g[big], o[big], rtol=1e-6)
    assert (g[~big] < 2 * tiny).all()
    exact = float(np.mean(g == o))
    anc = torch.zeros(R, dtype=torch.int32, device="cuda")
    y = torch.zeros((R, gamma), dtype=torch.int32, device="cuda")
    K = (R * gamma) // 3
    s = {k: v.cpu().numpy() for k, v in ds.dspark_schedule(c, K, anc, y).items()}
    os_ = oracle.schedule(g, K, np.zeros(R, np.int32), np.zeros((R, gamma), np.int32))
    np.testing.assert_array_equal(s["l"], os_.l)
    np.testing.assert_array_equal(s["a"], os_.a)
    print(f"[sts apply R={R} gamma={gamma}] bit-identical fraction {exact:.4f}", flush=True)


def test_lagged_pipeline_over_steps():
    """The serving loop the pages describe, over five steps with fresh inputs
    each step: the confidence calibrated with temperatures fitted once
    (sequential temperature scaling), the capacity of step t taken from the
    survival of step t - 2 (fixed-length verify before that), then draft,
    schedule, verify.  Every stage is compared with the oracle on the same
    inputs the GPU stage received."""
    import torch
    import draft_verify_sampling_bias_amd as ds
    import oracle
    R, gamma, V, rank = 24, 5, 3000, 64
    zc, nc, _ = synth.make_calibration(960, 6000, gamma)
    tau = ds.dspark_sts_fit(torch.from_numpy(zc).cuda(), torch.from_numpy(nc).cuda())
    tau_np = tau.cpu().numpy()
    np.testing.assert_allclose(tau_np, oracle.sts_fit(zc, nc).tau.astype(np.float32), rtol=1e-6)
    sps = synth.sps_table(R * (gamma + 1) + 1, t_row=1.0 / 2048)
    sps_d = torch.from_numpy(sps).cuda()
    survival = {}
    for t in range(5):
        inp = synth.make_custom(970 + t, R, gamma, V, rank, policy="temps", name=f"loop{t}")
        z = synth.make_calibration(980 + t, R, gamma)[0]
        c = ds.dspark_sts_apply(torch.from_numpy(z).cuda(), tau)
        c_np = c.cpu().numpy()
        o_c = oracle.sts_apply(z, tau_np)
        np.testing.assert_allclose(c_np, o_c, rtol=1e-6, atol=2 * np.finfo(np.float32).tiny)
        inp.c = c_np                                  # the oracle schedules on the same confidence
        if t >= 2:
            cap = ds.dspark_capacity(torch.from_numpy(survival[t - 2]).cuda(), sps_d)
            K = int(cap["K"].cpu()[0])
            assert K == oracle.capacity(survival[t - 2], sps).K
        else:
            K = R * gamma
        d = upload(inp)
        g = gpu_step(d, K, gamma)
        tally = Tally()
        reqs = list(range(R))
        dr = compare_draft(inp, g, reqs, tally)
        compare_schedule(inp, g, K)
        compare_verify(inp, g, reqs, tally, dr)
        tally.check()
        survival[t] = g["a"]
        print(f"[loop step {t}] K={K} rows={int(g['row_offsets'][-1])} accepted={int(g['n_accept'].sum())} "
              f"{tally.summary()}", flush=True)


@pytest.mark.parametrize("R,gamma", [(5, 3), (64, 7), (300, 5), (1024, 16), (3000, 5)])
def test_schedule_ties(R, gamma):
    """Top-K schedule bit-exact against the oracle when survival values tie
    heavily (confidences from a small set, exact 0 and 1), at every capacity
    from none to all: the selection then depends on the (k, r) tie-break."""
    import torch
    import draft_verify_sampling_bias_amd as ds
    import oracle
    rng = np.random.default_rng(1100 + R + gamma)
    c = rng.choice(np.array([1.0, 1.0, 0.5, 0.25, 0.0], np.float32), (R, gamma))
    anc = rng.integers(0, 50000, R).astype(np.int32)
    y = rng.integers(0, 50000, (R, gamma)).astype(np.int32)
    cd, ad, yd = (torch.from_numpy(x).cuda() for x in (c, anc, y))
    n = R * gamma
    Ks = sorted({0, 1, R, n // 3, n // 2, n - 1, n, int(rng.integers(0, n + 1)), int(rng.integers(0, n + 1))})
    for K in Ks:
        g = {k: v.cpu().numpy() for k, v in ds.dspark_schedule(cd, K, ad, yd).items()}
        o = oracle.schedule(c, K, anc, y)
        np.testing.assert_array_equal(g["l"], o.l, err_msg=f"K={K}")
        np.testing.assert_array_equal(g["row_offsets"], o.row_offsets)
        for f in ("row_req", "row_pos", "row_tok"):
            np.testing.assert_array_equal(g[f], getattr(o, f), err_msg=f)


@pytest.mark.parametrize("head", ["markov", "rnn"])
def test_step_graph_capture_replays(head):
    """A whole step (draft, schedule, verify) captured once in a HIP graph.
    Every buffer is allocated before the capture and every call has a shape
    known on the host (the capacity is fixed ahead), so the captured step
    replays without host work.  The graph is replayed several times, with
    eager work and synchronisations in between, with new inputs copied in
    before each replay, and every replay must equal the eager step on the
    same inputs bit for bit.  With the RNN head (and the packed W2) the
    captured draft also packs A, runs the state kernel once and writes the
    states, which the verify reads."""
    import torch
    import draft_verify_sampling_bias_amd as ds
    R, gamma, V, rank = 64, 5, 20000, 128
    inps = [synth.make_custom(1200 + i, R, gamma, V, rank, policy="temps", name=f"graph{i}") for i in range(3)]
    K = (R * gamma) // 2
    d = upload(inps[0])
    rnn = head == "rnn"
    rk, vk = {}, {}
    if rnn:
        h_buf = torch.empty((R, gamma, rank), dtype=torch.float32, device="cuda:0")
        rk = dict(A=upload_A(synth.make_rnn_A(1200, rank), "bf16"), act=1, h=h_buf,
                  W2_packed=ds.dspark_pack_w2(d["W2"]))
        vk = dict(h=h_buf)
    # the schedule of these inputs decides which target rows the verify reads;
    # the rows buffer is refilled (eagerly) before each replay
    n_rows = ds.dspark_schedule_rows(R, gamma, K)
    dev = torch.device("cuda:0")
    y = torch.empty((R, gamma), dtype=torch.int32, device=dev)
    q_tok = torch.empty((R, gamma), dtype=torch.float32, device=dev)
    q_stats = torch.empty((R, gamma, 2), dtype=torch.float32, device=dev)
    ws_d = torch.empty(ds.draft_workspace_bytes(R, gamma, V, rank, ds.W_BF16, head=ds.HEAD_RNN if rnn else 0,
                                                act=1 if rnn else 0), dtype=torch.uint8, device=dev)
    sch = dict(a=torch.empty((R, gamma), dtype=torch.float32, device=dev),
               l=torch.empty(R, dtype=torch.int32, device=dev),
               row_offsets=torch.empty(R + 1, dtype=torch.int32, device=dev),
               row_req=torch.empty(n_rows, dtype=torch.int32, device=dev),
               row_pos=torch.empty(n_rows, dtype=torch.int32, device=dev),
               row_tok=torch.empty(n_rows, dtype=torch.int32, device=dev),
               expected_tokens=torch.empty(1, dtype=torch.float32, device=dev))
    rows = torch.empty((n_rows, V), dtype=torch.float32, device=dev)
    n_acc = torch.empty(R, dtype=torch.int32, device=dev)
    out_tok = torch.empty(R, dtype=torch.int32, device=dev)
    p_tok = torch.empty((R, gamma), dtype=torch.float32, device=dev)
    ws_v = torch.empty(ds.verify_workspace_bytes(R, gamma, V, rank, ds.W_BF16, n_rows,
                                                 head=ds.HEAD_RNN if rnn else 0), dtype=torch.uint8, device=dev)

    def step():
        ds.dspark_draft_block(d["U"], d["W1"], d["W2"], d["anchor"], d["temp"], d["u_draft"],
                              out=(y, q_tok, q_stats), workspace=ws_d, **rk)
        ds.dspark_schedule(d["c"], K, d["anchor"], y, out=sch)
        ds.dspark_verify(rows, sch["row_offsets"], d["U"], d["W1"], d["W2"], d["anchor"], d["temp"], y, q_tok,
                         q_stats, d["u_accept"], d["u_final"], out=(n_acc, out_tok, p_tok), workspace=ws_v, **vk)

    def load(inp):
        nd = upload(inp)
        for k in d:
            d[k].copy_(nd[k])
        # the target rows of this input's schedule (stand-in for the target forward)
        ds.dspark_draft_block(d["U"], d["W1"], d["W2"], d["anchor"], d["temp"], d["u_draft"],
                              out=(y, q_tok, q_stats), workspace=ws_d, **rk)
        ds.dspark_schedule(d["c"], K, d["anchor"], y, out=sch)
        rows.copy_(d["target"][sch["row_req"].long(), sch["row_pos"].long()])
        torch.cuda.synchronize()

    def snapshot():
        torch.cuda.synchronize()
        return {k: v.clone() for k, v in dict(y=y, q_tok=q_tok, q_stats=q_stats, n_acc=n_acc, out_tok=out_tok,
                                               p_tok=p_tok, **sch, **vk).items()}

    load(inps[0])
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm the stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(6):
        inp = inps[rep % 3]
        load(inp)
        step()
        eager = snapshot()
        torch.sum(rows, dim=0)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        replay = snapshot()
        for k in eager:
            assert torch.equal(eager[k], replay[k]), (rep, k)
        print(f"[graph replay {rep} {head}] input {rep % 3}: identical to eager; accepted {int(n_acc.sum())}",
              flush=True)
