"""The C ABI on the host: libgdn.so loads, exports exactly what include/gdn.h
declares, and rejects bad arguments before enqueuing anything.  No GPU: every
call below fails validation, which runs before any HIP call, so the fake
device addresses are never dereferenced.
"""
import ctypes
import os
import re
import subprocess

import pytest

import gated_deltanet_layer_02_amd as gdn
from gated_deltanet_layer_02_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\*?\s+\*?(gdn_[a-z_]+)\s*\(", src, flags=re.M))


def test_library_exports_every_declared_symbol():
    decl = declared_functions()
    assert decl == set(B.EXPORTED), decl
    nm = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(gdn_\w+)", nm))
    assert decl <= exported, decl - exported
    lib = gdn.lib()
    for name in decl:
        assert getattr(lib, name) is not None


def test_status_strings():
    for code, name in B.STATUS_NAMES.items():
        assert gdn.gdn_status_string(code).startswith(name)
    assert "unknown" in gdn.gdn_status_string(99)


def test_workspace_size_grows_with_tokens():
    sizes = []
    for T in (0, 1, 64, 65, 4096, 65536):
        sizes.append(gdn.gdn_prefill_workspace_size(B.make_desc(1, T)))
    assert sizes == sorted(sizes) and sizes[-1] > sizes[0]
    # fp32 io doubles the fragment storage
    s_bf = gdn.gdn_prefill_workspace_size(B.make_desc(1, 4096, io_dtype=B.GDN_BF16))
    s_f = gdn.gdn_prefill_workspace_size(B.make_desc(1, 4096, io_dtype=B.GDN_F32))
    assert s_f > 1.9 * s_bf


def test_workspace_size_with_segments():
    """GDN_FLAG_SEGMENTS adds, for one sequence, room for up to 16 segments:
    31 + 15 state-sized buffers of Hv heads and the identity chains' bf16
    outputs of every token; descriptors of several sequences are unchanged."""
    T, Hv = 4096, 32
    plain = gdn.gdn_prefill_workspace_size(B.make_desc(1, T))
    seg = gdn.gdn_prefill_workspace_size(B.make_desc(1, T, segments=True))
    extra = (31 + 15) * Hv * 128 * 128 * 4 + T * Hv * 128 * 2
    assert extra <= seg - plain <= extra + 3 * 256
    assert gdn.gdn_prefill_workspace_size(B.make_desc(3, T, segments=True)) == \
        gdn.gdn_prefill_workspace_size(B.make_desc(3, T))
    # the default rule: one sequence of >= 32 chunks with <= 16 value heads,
    # unless separate launches are asked for alone
    few = dict(num_k_heads=2, num_v_heads=4)
    grow = gdn.gdn_prefill_workspace_size(B.make_desc(1, T, **few)) - \
        gdn.gdn_prefill_workspace_size(B.make_desc(1, T, separate_launches=True, **few))
    assert grow >= (31 + 15) * 4 * 128 * 128 * 4 + T * 4 * 128 * 2
    assert gdn.gdn_prefill_workspace_size(B.make_desc(1, 2047, **few)) == \
        gdn.gdn_prefill_workspace_size(B.make_desc(1, 2047, separate_launches=True, **few))


FAKE = 1 << 40          # 256-byte aligned fake device address; never dereferenced
STEP = 1 << 34          # distance between fake tensors (no overlaps)


def _ptrs(n, base=FAKE):
    return [base + i * STEP for i in range(n)]


def _prefill_rc(desc, **over):
    names = ["q", "k", "v", "g", "beta", "z", "conv_w", "norm_w", "cu", "S0", "cs_in", "out",
             "S1", "cs_out"]
    vals = dict(zip(names, _ptrs(len(names))))
    ws, ws_bytes = FAKE + 20 * STEP, 1 << 33
    vals.update({k: v for k, v in over.items() if k in vals})
    ws = over.get("ws", ws)
    ws_bytes = over.get("ws_bytes", ws_bytes)
    lib = gdn.lib()
    args = [vals[n] for n in names]
    return lib.gdn_prefill(ctypes.byref(desc), *args, ws, ws_bytes, None)


def test_prefill_validation_errors():
    cases = [
        (dict(num_seqs=0), {}, 2),
        (dict(num_k_heads=3), {}, 2),                    # 32 % 3 != 0
        (dict(total_tokens=-1), {}, 2),
        (dict(head_k_dim=64), {}, 3),
        (dict(head_v_dim=256), {}, 3),
        (dict(conv_kernel=3), {}, 3),
        (dict(flags=0x40), {}, 3),
        (dict(flags=0x3F), dict(ws_bytes=1024), 6),       # the launch-form and test flags are accepted
        (dict(io_dtype=5), {}, 4),
        (dict(state_dtype=B.GDN_BF16), {}, 4),           # gdn_prefill: fp32 state (gdn_prefill_ex: either)
        (dict(scale=float("nan")), {}, 9),
        (dict(l2_eps=-1.0), {}, 9),
        ({}, dict(q=None), 1),
        ({}, dict(beta=None), 1),
        ({}, dict(out=None), 1),
        ({}, dict(z=None), 1),                            # z without norm_w
        ({}, dict(cu=None), 1),                           # N = 2 needs cu_seqlens
        ({}, dict(q=FAKE + 8), 5),
        ({}, dict(ws=FAKE + 20 * STEP + 16), 5),          # workspace 256-byte alignment
        ({}, dict(ws_bytes=1024), 6),
        ({}, dict(ws=None), 6),
        ({}, dict(out=FAKE), 8),                          # out aliases q
        ({}, dict(S1=FAKE + 11 * STEP), 8),               # final_state aliases out
    ]
    for dover, pover, want in cases:
        dd = B.make_desc(2, 100)
        for k, v in dover.items():
            setattr(dd, k, v)
        rc = _prefill_rc(dd, **pover)
        assert rc == want, (dover, pover, rc, want)
    # NULL descriptor
    lib = gdn.lib()
    assert lib.gdn_prefill(None, *([None] * 14), None, 0, None) == 1
    # workspace-size query validates too
    n = ctypes.c_size_t()
    bad = B.make_desc(1, 10, head_dim=64)
    assert lib.gdn_prefill_workspace_size(ctypes.byref(bad), ctypes.byref(n)) == 3
    assert lib.gdn_prefill_workspace_size(ctypes.byref(B.make_desc(1, 10)), None) == 1


def test_wait_status_validation():
    """gdn_prefill_wait_status checks its arguments before it synchronises or
    copies anything."""
    lib = gdn.lib()
    f = ctypes.c_int32(-1)
    assert lib.gdn_prefill_wait_status(FAKE, 1 << 20, None, None) == 1              # NULL result
    assert lib.gdn_prefill_wait_status(None, 1 << 20, None, ctypes.byref(f)) == 6     # no workspace
    assert lib.gdn_prefill_wait_status(FAKE, 255, None, ctypes.byref(f)) == 6        # < 256 bytes
    assert lib.gdn_prefill_wait_status(FAKE + 16, 1 << 20, None, ctypes.byref(f)) == 5
    assert f.value == -1


def test_static_prefill_refusals():
    """gdn_prefill_static refuses a workspace argument and calls whose
    workspace would exceed its static scratch, before any HIP call."""
    lib = gdn.lib()
    p = _ptrs(20)
    a = B.PrefillArgs(q=p[0], k=p[1], v=p[2], g=p[3], beta=p[4], out=p[5], final_state=p[6],
                      workspace=p[7], workspace_bytes=1 << 20)
    d = B.make_desc(1, 4096)
    assert lib.gdn_prefill_static(ctypes.byref(d), ctypes.byref(a), None) == 9          # workspace given
    a.workspace, a.workspace_bytes = None, 0
    assert lib.gdn_prefill_static(ctypes.byref(d), None, None) == 1
    # the limit: T_total / 64 + N chunk slots within GDN_STATIC_SCRATCH_BYTES
    big = B.make_desc(1, 64 * 73)
    assert gdn.gdn_prefill_workspace_size(big) > B.STATIC_SCRATCH_BYTES
    assert gdn.gdn_prefill_workspace_size(B.make_desc(1, 4671)) <= B.STATIC_SCRATCH_BYTES
    assert lib.gdn_prefill_static(ctypes.byref(big), ctypes.byref(a), None) == 6
    bad = B.make_desc(1, 4096, head_dim=64)
    assert lib.gdn_prefill_static(ctypes.byref(bad), ctypes.byref(a), None) == 3


def test_prefill_profiled_needs_events():
    d = B.make_desc(1, 10)
    lib = gdn.lib()
    rc = lib.gdn_prefill_profiled(ctypes.byref(d), *_ptrs(14), FAKE + 20 * STEP, 1 << 33, None,
                                  None, 8, None, None)
    assert rc == 1


def _decode_rc(desc, num_slots=None, **over):
    names = ["q", "k", "v", "g", "beta", "z", "conv_w", "norm_w", "state", "cs", "slots"]
    vals = dict(zip(names, _ptrs(len(names))))
    vals["slots"] = None
    vals.update({k: v for k, v in over.items() if k in vals})
    out = over.get("out", FAKE + 30 * STEP)
    lib = gdn.lib()
    ns = desc.num_seqs if num_slots is None else num_slots
    return lib.gdn_decode(ctypes.byref(desc), *[vals[n] for n in names], ns, out, None)


def test_decode_validation_errors():
    cases = [
        (dict(total_tokens=5), {}, None, 2),             # decode: T_total == N
        (dict(head_k_dim=96), {}, None, 3),
        (dict(state_dtype=7), {}, None, 4),
        ({}, dict(state=None), None, 1),
        ({}, dict(q=None), None, 1),
        ({}, dict(norm_w=None), None, 1),
        ({}, dict(v=FAKE + 4), None, 5),
        ({}, {}, 3, 2),                                    # fewer slots than sequences
        ({}, dict(out=FAKE + 8 * STEP), None, 8),         # out aliases the state
        ({}, dict(cs=FAKE + 8 * STEP), None, 8),          # conv state aliases the state
    ]
    for dover, pover, ns, want in cases:
        d = B.make_desc(4, 4, state_dtype=B.GDN_BF16)
        for k, v in dover.items():
            setattr(d, k, v)
        rc = _decode_rc(d, ns, **pover)
        assert rc == want, (dover, pover, rc, want)


def _ex_rc(desc, **over):
    """gdn_prefill_ex with fake, non-overlapping device pointers."""
    names = ["q", "k", "v", "g", "beta", "z", "conv_w", "norm_w", "cu_seqlens", "initial_state",
             "final_state", "conv_state_in", "conv_state_out", "state_slots", "state_snapshots",
             "snapshot_base", "out", "workspace"]
    vals = dict(zip(names, _ptrs(len(names))))
    vals.update(state_slots=None, state_snapshots=None, snapshot_base=None)
    ints = dict(num_state_slots=0, snapshot_every=0, num_snapshot_slots=0, workspace_bytes=1 << 33)
    for k, v in over.items():
        (vals if k in vals else ints)[k] = v
    a = B.PrefillArgs(**vals, **ints)
    return gdn.lib().gdn_prefill_ex(ctypes.byref(desc), ctypes.byref(a), None)


def test_prefill_ex_validation_errors():
    snap = dict(state_snapshots=FAKE + 30 * STEP, snapshot_base=FAKE + 31 * STEP, snapshot_every=2,
                num_snapshot_slots=8)
    cases = [
        ({}, dict(q=None), 1),
        ({}, dict(num_state_slots=1), 2),                         # fewer rows than sequences
        ({}, dict(state_slots=FAKE + 32 * STEP, num_state_slots=-1), 2),
        ({}, dict(snap, snapshot_base=None), 1),                  # snapshots need their rows
        ({}, dict(snap, snapshot_every=0), 2),
        ({}, dict(snap, num_snapshot_slots=0), 2),
        ({}, dict(snap, state_snapshots=FAKE + 16 * STEP), 8),    # snapshots alias out
        ({}, dict(snap, state_snapshots=FAKE + 9 * STEP), 8),     # ... the initial state
        ({}, dict(snap, state_snapshots=FAKE + 30 * STEP + 8), 5),
        ({}, dict(state_slots=FAKE + 32 * STEP + 4), 5),
        (dict(state_dtype=7), {}, 4),
    ]
    for dover, pover, want in cases:
        dd = B.make_desc(2, 100, state_dtype=B.GDN_BF16)
        for k, v in dover.items():
            setattr(dd, k, v)
        rc = _ex_rc(dd, **pover)
        assert rc == want, (dover, pover, rc, want)
    assert gdn.lib().gdn_prefill_ex(ctypes.byref(B.make_desc(1, 1)), None, None) == 1


def test_prefill_args_layout_matches_the_header(tmp_path):
    """The ctypes mirror of gdn_prefill_args has the C compiler's layout."""
    fields = [f for f, _ in B.PrefillArgs._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include "gdn.h"\n#include <stdio.h>\n#include <stddef.h>\nint main(void) {\n'
                   '  printf("%zu", sizeof(gdn_prefill_args));\n'
                   + "".join(f'  printf(" %zu", offsetof(gdn_prefill_args, {f}));\n' for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    "-D__HIP_PLATFORM_AMD__", str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    want = [ctypes.sizeof(B.PrefillArgs)] + [getattr(B.PrefillArgs, f).offset for f in fields]
    assert got == want


def test_verify_and_commit_validation_errors():
    lib = gdn.lib()
    P = _ptrs(15)

    def verify(desc, D=4, **over):
        names = ["q", "k", "v", "g", "beta", "z", "conv_w", "norm_w", "state", "cs", "slots",
                 "ckpt", "cck", "out"]
        vals = dict(zip(names, P))
        vals["slots"] = None
        vals.update(over)
        ns = over.get("ns", desc.num_seqs)
        return lib.gdn_decode_verify(ctypes.byref(desc), D, *[vals[n] for n in names[:11]], ns,
                                     vals["ckpt"], vals["cck"], vals["out"], None)

    d = B.make_desc(2, 8)
    assert verify(d, D=0) == 2
    assert verify(d, D=9) == 2
    assert verify(B.make_desc(2, 7)) == 2                      # total_tokens != N * D
    assert verify(d, q=None) == 1
    assert verify(d, ckpt=None) == 1
    assert verify(d, ns=1) == 2
    assert verify(d, ckpt=FAKE + 8 * STEP) == 8                 # checkpoints alias the state
    assert verify(d, out=FAKE + 11 * STEP) == 8                 # out aliases the checkpoints
    assert verify(d, cck=FAKE + 12 * STEP + 4) == 5

    def commit(desc, D=4, **over):
        vals = dict(ckpt=P[0], cck=P[1], acc=P[2], state=P[3], cs=P[4], slots=None)
        vals.update(over)
        ns = over.get("ns", desc.num_seqs)
        return lib.gdn_decode_commit(ctypes.byref(desc), D, vals["ckpt"], vals["cck"], vals["acc"],
                                     vals["state"], vals["cs"], vals["slots"], ns, None)

    assert commit(d, D=0) == 2
    assert commit(d, acc=None) == 1
    assert commit(d, state=P[0]) == 8                           # state pool aliases checkpoints
    assert commit(d, ns=1) == 2
