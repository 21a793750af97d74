"""CPU tests of the C ABI: the library loads, exports every function that
include/dspark.h declares, and rejects invalid arguments on the host before
enqueuing anything (no GPU is touched: every call here fails validation or is
a host-only query)."""
import ctypes
import os
import re
import subprocess

import pytest

import draft_verify_sampling_bias_amd as ds

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")

FAKE = 0x10000  # 64 KiB-aligned non-NULL address; never dereferenced by failing calls


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(dspark_\w+)\s*\(", txt, re.M)))


def test_header_declares_and_library_exports_everything():
    names = _declared()
    assert set(names) == set(ds.EXPORTED_SYMBOLS), names
    lib = ds.get_lib()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", ds.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(names) <= exported


def test_abi_version_and_strings():
    assert ds.dspark_abi_version() == ds.ABI_VERSION == 3
    strings = [ds.dspark_status_string(s) for s in range(10)]
    assert all(strings) and len(set(strings)) == 10
    assert "unknown status" not in strings
    assert ds.dspark_status_string(123) == "unknown status"


def test_schedule_rows():
    assert ds.dspark_schedule_rows(64, 7, 448) == 64 + 448
    assert ds.dspark_schedule_rows(64, 7, 10 ** 12) == 64 + 448
    assert ds.dspark_schedule_rows(256, 5, 300) == 556
    assert ds.dspark_schedule_rows(8, 3, -5) == 8
    assert ds.dspark_schedule_rows(0, 3, 5) == 0
    assert ds.dspark_schedule_rows(-1, 3, 5) == -1
    assert ds.dspark_schedule_rows(4, 0, 5) == -1


def test_workspace_sizes_match_struct_layout():
    # a struct_size mismatch would return DSPARK_ERR_ABI
    def up(x):
        return (x + 255) // 256 * 256

    H = ds.WORKSPACE_HEADER  # the error word (and arrival counters) come first
    assert H == 256
    # one (max, sum) record of two floats per (request row, 16-row segment);
    # the 16-row path (bf16 weights, R <= 64) always holds 64 request rows
    assert ds.draft_workspace_bytes(64, 7, 151936, 512, 1) == H + up(64 * 9496 * 8)
    assert ds.draft_workspace_bytes(3, 7, 1000, 64, 1) == H + up(64 * 63 * 8)
    # the input checks need no more room than the header
    assert ds.draft_workspace_bytes(3, 7, 1000, 64, 1, ds.CHECK_INPUTS) == H + up(64 * 63 * 8)
    # 64-row segments above 64 requests (bf16): R + 17 record rows (padding
    # requests of the last chunk, one dummy row)
    assert ds.draft_workspace_bytes(65, 7, 151936, 512, 1) == H + up((65 + 17) * 2374 * 8)
    # 32-row segments, one row per request, for fp32 weights
    assert ds.draft_workspace_bytes(65, 7, 151936, 512, 0) == H + up(65 * 4748 * 8)
    assert ds.draft_workspace_bytes(8, 7, 1024, 32, 0) == H + up(8 * 32 * 8)
    # the RNN head (16-row path) also holds A in the fragment-packed layout:
    # ceil(rank / 16) segments x rank / 32 k-steps x 1 KiB (rank 64: 2 k-steps)
    assert ds.draft_workspace_bytes(64, 7, 151936, 512, 1, head=ds.HEAD_RNN, act=1) == \
        H + up(64 * 9496 * 8) + 32 * 16 * 1024
    assert ds.draft_workspace_bytes(3, 7, 1000, 64, 1, head=ds.HEAD_RNN, act=0) == H + up(64 * 63 * 8) + 4 * 2 * 1024
    assert ds.dspark_w2_packed_bytes(512, 512) == 32 * 16 * 1024
    # verify: chunk records (16 bytes per 4096-entry chunk of each target row),
    # residual info/stats, then the residual segment records
    nb = ds.verify_workspace_bytes(64, 7, 151936, 512, 1, 512)
    assert nb == H + up(512 * 38 * 16) + up(64 * 16) + up(64 * 16) + up(64 * 9496 * 8)
    # 64-row path: plus the count and list (48 bytes per request) of the
    # requests that need the residual pass
    nb = ds.verify_workspace_bytes(256, 5, 129280, 512, 1, 768)
    assert nb == (H + up(768 * 32 * 16) + up(256 * 16) + up(256 * 16) + up((256 + 17) * 2020 * 8) + up(4)
                  + up(256 * 48))
    # the schedule calls need a workspace (the header) only for the checks
    assert ds.dspark_schedule_workspace_size(64, 7) == 0
    assert ds.dspark_schedule_workspace_size(64, 7, ds.CHECK_INPUTS) == H
    assert ds.dspark_cutoff_workspace_size(1024, 16) == 0
    assert ds.dspark_cutoff_workspace_size(1024, 16, ds.CHECK_INPUTS) == H


def _draft_args(**kw):
    base = dict(struct_size=ctypes.sizeof(ds.DraftArgs), R=4, gamma=3, V=1000, rank=64, wdtype=1,
                U=FAKE, W1=FAKE, W2=FAKE, anchor=FAKE, temp=FAKE, u_draft=FAKE, y=FAKE, q_tok=FAKE,
                q_stats=FAKE, workspace=None, workspace_bytes=0, stream=None, prof_events=None)
    base.update(kw)
    return ds.DraftArgs(**base)


def _call(fn, args):
    return getattr(ds.get_lib(), fn)(ctypes.byref(args))


@pytest.mark.parametrize("kw,status", [
    (dict(struct_size=8), ds.Status.ERR_ABI),
    (dict(R=-1), ds.Status.ERR_SHAPE),
    (dict(gamma=0), ds.Status.ERR_SHAPE),
    (dict(gamma=17), ds.Status.ERR_UNSUPPORTED),
    (dict(V=0), ds.Status.ERR_SHAPE),
    (dict(rank=12), ds.Status.ERR_UNSUPPORTED),
    (dict(rank=520), ds.Status.ERR_UNSUPPORTED),
    (dict(wdtype=7), ds.Status.ERR_DTYPE),
    (dict(U=None), ds.Status.ERR_NULL),
    (dict(q_stats=None), ds.Status.ERR_NULL),
    (dict(U=FAKE + 4), ds.Status.ERR_ALIGN),
    (dict(W2=FAKE + 8), ds.Status.ERR_ALIGN),
    (dict(), ds.Status.ERR_WORKSPACE),
    (dict(workspace=FAKE, workspace_bytes=100), ds.Status.ERR_WORKSPACE),
    (dict(workspace=FAKE + 64, workspace_bytes=1 << 30), ds.Status.ERR_ALIGN),
    (dict(flags=2), ds.Status.ERR_UNSUPPORTED),            # unknown flag bit
    (dict(flags=1 << 31), ds.Status.ERR_UNSUPPORTED),
    # the RNN head: known head and activation, the 16-row path only
    (dict(head=2), ds.Status.ERR_UNSUPPORTED),
    (dict(head=1, act=2, A=FAKE, h=FAKE), ds.Status.ERR_UNSUPPORTED),
    (dict(head=1, A=FAKE, h=FAKE, R=65), ds.Status.ERR_UNSUPPORTED),      # 64-row path
    (dict(head=1, A=FAKE, h=FAKE, wdtype=0), ds.Status.ERR_UNSUPPORTED),  # fp32 path
    (dict(head=1, A=None, h=FAKE), ds.Status.ERR_NULL),
    (dict(head=1, A=FAKE, h=None), ds.Status.ERR_NULL),
    (dict(head=1, A=FAKE + 8, h=FAKE), ds.Status.ERR_ALIGN),
    (dict(head=1, A=FAKE, h=FAKE + 4), ds.Status.ERR_ALIGN),
    (dict(head=1, A=FAKE, h=FAKE), ds.Status.ERR_WORKSPACE),  # valid RNN arguments up to the workspace
])
def test_draft_rejects_invalid_arguments(kw, status):
    assert _call("dspark_draft_block", _draft_args(**kw)) == status


def test_zero_requests_is_a_noop():
    assert _call("dspark_draft_block", _draft_args(R=0, U=None, W1=None)) == ds.Status.OK
    a = ds.ScheduleArgs(struct_size=ctypes.sizeof(ds.ScheduleArgs), R=0, gamma=3, K=5)
    assert _call("dspark_schedule", a) == ds.Status.OK
    v = ds.VerifyArgs(struct_size=ctypes.sizeof(ds.VerifyArgs), R=0, gamma=3, V=100, rank=8, wdtype=1, n_rows=0)
    assert _call("dspark_verify", v) == ds.Status.OK


def _verify_args(**kw):
    base = dict(struct_size=ctypes.sizeof(ds.VerifyArgs), R=4, gamma=3, V=1000, rank=64, wdtype=1, n_rows=16,
                workspace=None, workspace_bytes=0, stream=None)
    for f in ("target", "row_offsets", "U", "W1", "W2", "anchor", "temp", "y", "q_tok", "q_stats", "u_accept",
              "u_final", "n_accept", "out_tok", "p_tok"):
        base[f] = FAKE
    base.update(kw)
    return ds.VerifyArgs(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(struct_size=4), ds.Status.ERR_ABI),
    (dict(n_rows=3), ds.Status.ERR_SHAPE),
    (dict(n_rows=17), ds.Status.ERR_SHAPE),
    (dict(target=None), ds.Status.ERR_NULL),
    (dict(u_final=None), ds.Status.ERR_NULL),
    (dict(target=FAKE + 4), ds.Status.ERR_ALIGN),
    (dict(q_stats=FAKE + 4), ds.Status.ERR_ALIGN),
    (dict(), ds.Status.ERR_WORKSPACE),
    (dict(flags=4), ds.Status.ERR_UNSUPPORTED),
    (dict(head=3), ds.Status.ERR_UNSUPPORTED),
    (dict(head=1, h=FAKE, R=65, n_rows=65), ds.Status.ERR_UNSUPPORTED),
    (dict(head=1, h=FAKE, wdtype=0), ds.Status.ERR_UNSUPPORTED),
    (dict(head=1, h=None), ds.Status.ERR_NULL),
    (dict(head=1, h=FAKE + 4), ds.Status.ERR_ALIGN),
    (dict(head=1, h=FAKE), ds.Status.ERR_WORKSPACE),
])
def test_verify_rejects_invalid_arguments(kw, status):
    assert _call("dspark_verify", _verify_args(**kw)) == status


@pytest.mark.parametrize("kw,status", [
    (dict(struct_size=0), ds.Status.ERR_ABI),
    (dict(gamma=0), ds.Status.ERR_SHAPE),
    (dict(R=1025, gamma=9), ds.Status.ERR_UNSUPPORTED),   # ceil(R/1024) * gamma > 16
    (dict(c=None), ds.Status.ERR_NULL),
    (dict(row_tok=FAKE + 2), ds.Status.ERR_ALIGN),
    (dict(flags=2), ds.Status.ERR_UNSUPPORTED),
    # the input checks write their error word into a workspace
    (dict(flags=1), ds.Status.ERR_WORKSPACE),
    (dict(flags=1, workspace=FAKE, workspace_bytes=255), ds.Status.ERR_WORKSPACE),
    (dict(flags=1, workspace=FAKE + 128, workspace_bytes=256), ds.Status.ERR_ALIGN),
])
def test_schedule_rejects_invalid_arguments(kw, status):
    base = dict(struct_size=ctypes.sizeof(ds.ScheduleArgs), R=8, gamma=4, K=10)
    for f in ("c", "anchor", "y", "a", "l", "row_offsets", "row_req", "row_pos", "row_tok"):
        base[f] = FAKE
    base.update(kw)
    assert _call("dspark_schedule", ds.ScheduleArgs(**base)) == status


@pytest.mark.parametrize("kw,status", [
    (dict(struct_size=0), ds.Status.ERR_ABI),
    (dict(gamma=0), ds.Status.ERR_SHAPE),
    (dict(conf_min=float("nan")), ds.Status.ERR_SHAPE),
    (dict(R=-2), ds.Status.ERR_SHAPE),
    (dict(gamma=17), ds.Status.ERR_UNSUPPORTED),
    (dict(R=1025, gamma=9), ds.Status.ERR_UNSUPPORTED),
    (dict(y=None), ds.Status.ERR_NULL),
    (dict(row_pos=FAKE + 2), ds.Status.ERR_ALIGN),
    (dict(flags=8), ds.Status.ERR_UNSUPPORTED),
    (dict(flags=1), ds.Status.ERR_WORKSPACE),
])
def test_cutoff_rejects_invalid_arguments(kw, status):
    base = dict(struct_size=ctypes.sizeof(ds.CutoffArgs), R=8, gamma=4, conf_min=0.5)
    for f in ("c", "anchor", "y", "a", "l", "row_offsets", "row_req", "row_pos", "row_tok"):
        base[f] = FAKE
    base.update(kw)
    assert _call("dspark_schedule_cutoff", ds.CutoffArgs(**base)) == status
    assert _call("dspark_schedule_cutoff", ds.CutoffArgs(struct_size=ctypes.sizeof(ds.CutoffArgs), R=0, gamma=3,
                                                         conf_min=0.5)) == ds.Status.OK


@pytest.mark.parametrize("kw,status", [
    (dict(struct_size=8), ds.Status.ERR_ABI),
    (dict(gamma=0), ds.Status.ERR_SHAPE),
    (dict(R=-1), ds.Status.ERR_SHAPE),
    (dict(gamma=17), ds.Status.ERR_UNSUPPORTED),
    (dict(R=1025, gamma=16), ds.Status.ERR_UNSUPPORTED),    # R * gamma > 16384
    (dict(n_sps=8), ds.Status.ERR_SHAPE),                    # n_sps < R + 1
    (dict(a_lag=None), ds.Status.ERR_NULL),
    (dict(sps=None), ds.Status.ERR_NULL),
    (dict(K=None), ds.Status.ERR_NULL),
    (dict(sps=FAKE + 2), ds.Status.ERR_ALIGN),
    (dict(expected=FAKE + 4), ds.Status.ERR_ALIGN),
    (dict(theta=FAKE + 4), ds.Status.ERR_ALIGN),
])
def test_capacity_rejects_invalid_arguments(kw, status):
    base = dict(struct_size=ctypes.sizeof(ds.CapacityArgs), R=8, gamma=4, n_sps=41, a_lag=FAKE, sps=FAKE, K=FAKE)
    base.update(kw)
    assert _call("dspark_capacity", ds.CapacityArgs(**base)) == status


def test_capacity_largest_batch_passes_the_size_checks():
    # R * gamma = 16384 exactly and n_sps = R + 1 are inside the limits: with a
    # NULL K the call must fail on the pointer check, not on a size check
    a = ds.CapacityArgs(struct_size=ctypes.sizeof(ds.CapacityArgs), R=1024, gamma=16, n_sps=1025,
                        a_lag=FAKE, sps=FAKE, K=None)
    assert _call("dspark_capacity", a) == ds.Status.ERR_NULL


@pytest.mark.parametrize("kw,status", [
    (dict(struct_size=4), ds.Status.ERR_ABI),
    (dict(N=-1), ds.Status.ERR_SHAPE),
    (dict(gamma=0), ds.Status.ERR_SHAPE),
    (dict(gamma=17), ds.Status.ERR_UNSUPPORTED),
    (dict(z=None), ds.Status.ERR_NULL),
    (dict(n_acc=None), ds.Status.ERR_NULL),
    (dict(tau=None), ds.Status.ERR_NULL),
    (dict(tau=FAKE + 1), ds.Status.ERR_ALIGN),
])
def test_sts_fit_rejects_invalid_arguments(kw, status):
    base = dict(struct_size=ctypes.sizeof(ds.StsFitArgs), N=100, gamma=5, z=FAKE, n_acc=FAKE, tau=FAKE)
    base.update(kw)
    assert _call("dspark_sts_fit", ds.StsFitArgs(**base)) == status


@pytest.mark.parametrize("kw,status", [
    (dict(struct_size=4), ds.Status.ERR_ABI),
    (dict(R=-1), ds.Status.ERR_SHAPE),
    (dict(gamma=0), ds.Status.ERR_SHAPE),
    (dict(gamma=17), ds.Status.ERR_UNSUPPORTED),
    (dict(z=None), ds.Status.ERR_NULL),
    (dict(c=None), ds.Status.ERR_NULL),
    (dict(c=FAKE + 2), ds.Status.ERR_ALIGN),
])
def test_sts_apply_rejects_invalid_arguments(kw, status):
    base = dict(struct_size=ctypes.sizeof(ds.StsApplyArgs), R=8, gamma=5, z=FAKE, tau=FAKE, c=FAKE)
    base.update(kw)
    assert _call("dspark_sts_apply", ds.StsApplyArgs(**base)) == status
    # nothing to do for an empty batch
    assert _call("dspark_sts_apply", ds.StsApplyArgs(struct_size=ctypes.sizeof(ds.StsApplyArgs), R=0,
                                                     gamma=5)) == ds.Status.OK


def test_packed_w2_bytes():
    # ceil(V/16) segments x k-steps (2/4/8/16 for rank <= 64/128/256/512) x 1 KiB
    assert ds.dspark_w2_packed_bytes(151936, 512) == 9496 * 16 * 1024
    assert ds.dspark_w2_packed_bytes(1000, 96) == 63 * 4 * 1024
    assert ds.dspark_w2_packed_bytes(5, 8) == 1 * 2 * 1024
    assert ds.dspark_w2_packed_bytes(0, 64) == 0
    assert ds.dspark_w2_packed_bytes(100, 12) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(struct_size=4), ds.Status.ERR_ABI),
    (dict(rank=520), ds.Status.ERR_UNSUPPORTED),
    (dict(V=0), ds.Status.ERR_SHAPE),
    (dict(W2=None), ds.Status.ERR_NULL),
    (dict(W2_packed=FAKE + 8), ds.Status.ERR_ALIGN),
    (dict(W2_packed_bytes=63 * 4 * 1024 - 1), ds.Status.ERR_WORKSPACE),
])
def test_pack_rejects_invalid_arguments(kw, status):
    base = dict(struct_size=ctypes.sizeof(ds.PackArgs), V=1000, rank=96, W2=FAKE, W2_packed=FAKE,
                W2_packed_bytes=63 * 4 * 1024)
    base.update(kw)
    assert _call("dspark_pack_w2", ds.PackArgs(**base)) == status


def test_packed_w2_needs_bf16_alignment_and_size():
    big = dict(workspace=FAKE, workspace_bytes=1 << 30)
    need = ds.dspark_w2_packed_bytes(1000, 64)
    assert _call("dspark_draft_block", _draft_args(wdtype=0, W2_packed=FAKE, W2_packed_bytes=need,
                                                   **big)) == ds.Status.ERR_DTYPE
    assert _call("dspark_draft_block", _draft_args(W2_packed=FAKE + 4, W2_packed_bytes=need,
                                                   **big)) == ds.Status.ERR_ALIGN
    assert _call("dspark_verify", _verify_args(wdtype=0, W2_packed=FAKE, W2_packed_bytes=need,
                                               **big)) == ds.Status.ERR_DTYPE
    # a packed copy smaller than the layout of (V, rank) is rejected: made for
    # a smaller V or rank, it would be read past its end
    for fn, mk in (("dspark_draft_block", _draft_args), ("dspark_verify", _verify_args)):
        assert _call(fn, mk(W2_packed=FAKE, W2_packed_bytes=need - 1, **big)) == ds.Status.ERR_WORKSPACE
        assert _call(fn, mk(W2_packed=FAKE, W2_packed_bytes=0, **big)) == ds.Status.ERR_WORKSPACE
        assert _call(fn, mk(W2_packed=FAKE, W2_packed_bytes=ds.dspark_w2_packed_bytes(900, 64),
                            **big)) == ds.Status.ERR_WORKSPACE


def test_check_needs_a_workspace():
    lib = ds.get_lib()
    bits = ctypes.c_uint32(7)
    assert lib.dspark_check(None, None, ctypes.byref(bits)) == ds.Status.ERR_NULL
    assert bits.value == 7  # untouched on error


def test_binding_checks_the_packed_copy():
    """The binding refuses a packed copy of the wrong type, device, layout or
    size before calling the library (CPU tensors: nothing is launched)."""
    import torch
    dev = torch.device("cpu")
    need = ds.dspark_w2_packed_bytes(1000, 64)
    assert ds._w2_packed(None, dev, 1000, 64) == (None, 0)
    with pytest.raises(TypeError):
        ds._w2_packed(torch.zeros(need, dtype=torch.int16), dev, 1000, 64)
    with pytest.raises(ValueError):
        ds._w2_packed(torch.zeros(need - 1, dtype=torch.uint8), dev, 1000, 64)
    with pytest.raises(ValueError):
        ds._w2_packed(torch.zeros(2 * need, dtype=torch.uint8)[::2], dev, 1000, 64)
    ptr, nbytes = ds._w2_packed(torch.zeros(need, dtype=torch.uint8), dev, 1000, 64)
    assert nbytes == need and ptr


def test_null_args_pointer():
    lib = ds.get_lib()
    n = ctypes.c_size_t(0)
    assert lib.dspark_schedule_workspace_size(None, ctypes.byref(n)) == ds.Status.ERR_NULL
    assert lib.dspark_cutoff_workspace_size(None, ctypes.byref(n)) == ds.Status.ERR_NULL
    assert lib.dspark_draft_block(None) == ds.Status.ERR_NULL
    assert lib.dspark_verify(None) == ds.Status.ERR_NULL
    assert lib.dspark_schedule(None) == ds.Status.ERR_NULL
    assert lib.dspark_schedule_cutoff(None) == ds.Status.ERR_NULL
    assert lib.dspark_capacity(None) == ds.Status.ERR_NULL
    assert lib.dspark_sts_fit(None) == ds.Status.ERR_NULL
    assert lib.dspark_sts_apply(None) == ds.Status.ERR_NULL


def test_binding_fails_loudly_without_the_library(tmp_path):
    """No fallback: with libdspark.so absent, the binding's first use raises
    ImportError (run in a child process against a copy of the package whose
    library is missing, so the loaded library of this process is untouched)."""
    import shutil
    import sys
    pkg = os.path.join(ROOT, "draft_verify_sampling_bias_amd")
    dst = tmp_path / "draft_verify_sampling_bias_amd"
    shutil.copytree(pkg, dst, ignore=shutil.ignore_patterns("*.so", "_build", "__pycache__"))
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import draft_verify_sampling_bias_amd as ds\n"
            "assert not ds.LIB_PATH.startswith(%r)\n"
            "try:\n"
            "    ds.dspark_abi_version()\n"
            "except ImportError as e:\n"
            "    print('raised', e)\n"
            "else:\n"
            "    raise SystemExit('no error')\n") % (str(tmp_path), ROOT + os.sep)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=str(tmp_path))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "raised" in r.stdout and "libdspark.so" in r.stdout


def test_header_is_plain_c(tmp_path):
    """include/dspark.h is a C header: it compiles as C99 with -pedantic and
    as C++17, with no warnings."""
    import shutil
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    for compiler, lang, std in (("gcc", "c", "c99"), ("g++", "c++", "c++17")):
        if shutil.which(compiler) is None:
            pytest.skip(f"{compiler} not installed")
        src = tmp_path / f"t.{lang}"
        src.write_text('#include "dspark.h"\nint main(void) { return 0; }\n')
        r = subprocess.run([compiler, "-x", lang, f"-std={std}", "-Wall", "-Wextra", "-Werror", "-pedantic",
                            "-fsyntax-only", "-I", inc, str(src)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_noalloc_draft_refuses_before_enqueuing():
    """dspark_draft_block_noalloc: the size checks of dspark_draft_block, then
    the static workspace's limit and the refusal of the input checks, all on
    the host (fake pointers: none of these calls may reach a launch)."""
    assert ds.NOALLOC_SCRATCH_BYTES == 64 << 20
    fn = "dspark_draft_block_noalloc"
    assert _call(fn, _draft_args(struct_size=8)) == ds.Status.ERR_ABI
    assert _call(fn, _draft_args(gamma=0)) == ds.Status.ERR_SHAPE
    assert _call(fn, _draft_args(R=0)) == ds.Status.OK
    assert _call(fn, _draft_args(flags=ds.CHECK_INPUTS)) == ds.Status.ERR_UNSUPPORTED
    # 16-row path: 512 bytes of records per 16 vocabulary entries + the header
    assert ds.draft_workspace_bytes(64, 7, 2097136, 512, 1) <= ds.NOALLOC_SCRATCH_BYTES
    big = 2097152
    assert ds.draft_workspace_bytes(64, 7, big, 512, 1) > ds.NOALLOC_SCRATCH_BYTES
    assert _call(fn, _draft_args(R=64, gamma=7, V=big, rank=512)) == ds.Status.ERR_WORKSPACE
    # 64-row path: R = 1024 at V = 129280 fits, R = 8192 does not
    assert ds.draft_workspace_bytes(1024, 5, 129280, 512, 1) <= ds.NOALLOC_SCRATCH_BYTES
    assert ds.draft_workspace_bytes(8192, 5, 129280, 512, 1) > ds.NOALLOC_SCRATCH_BYTES
    assert _call(fn, _draft_args(R=8192, gamma=5, V=129280, rank=512)) == ds.Status.ERR_WORKSPACE
    assert ds.get_lib().dspark_draft_block_noalloc(None) == ds.Status.ERR_NULL
