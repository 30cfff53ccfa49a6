"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point include/o1.h declares, and rejects invalid arguments before
touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "o1.h")


def _lib():
    import streaming_nystr_attention_amd as P

    if not os.path.exists(P.LIB_PATH):
        from streaming_nystr_attention_amd import build

        build.build()
    return P, P.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(o1_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("o1_create_groups", "o1_prefill", "o1_step", "o1_destroy_groups"):
        assert n in names


def test_library_exports_every_declared_symbol():
    P, L = _lib()
    names = declared_functions()
    out = subprocess.run(["nm", "-D", "--defined-only", P.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(P.EXPORTS) == set(names)
    for n in names:
        assert hasattr(L, n)


def test_abi_version():
    P, L = _lib()
    assert P.o1_abi_version() == 3


def _header_enum(prefix):
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return {n: int(v) for n, v in re.findall(rf"\b({prefix}[A-Z_0-9]+)\s*=\s*(\d+)", text)}


def test_binding_constants_match_the_header():
    P, _ = _lib()
    status = _header_enum("O1_E")
    assert re.search(r"\bO1_OK\s*=\s*0\b", open(HEADER).read()) and P.O1_OK == 0
    assert len(status) == 7
    for name, val in status.items():
        assert getattr(P, name) == val, name
    fields = _header_enum("O1_FIELD_")
    for name, val in fields.items():
        assert getattr(P, name[3:]) == val, name
    fold = re.search(r"#define\s+O1_FOLD_PERIOD\s+(\d+)", open(HEADER).read())
    assert fold and int(fold.group(1)) == P.FOLD_PERIOD
    for struct in ("o1_config", "o1_info"):
        body = re.search(rf"typedef struct {struct} \{{(.*?)\}} {struct};", open(HEADER).read(), re.S)
        decls = re.findall(r"(u?int\d+_t|double|float)\s+([\w\s,]+);",
                           re.sub(r"/\*.*?\*/", "", body.group(1), flags=re.S))
        ctype = {"int32_t": ctypes.c_int32, "int64_t": ctypes.c_int64, "uint64_t": ctypes.c_uint64,
                 "double": ctypes.c_double, "float": ctypes.c_float}
        fields = [(n.strip(), ctype[t]) for t, names in decls for n in names.split(",")]
        assert fields == list(getattr(P, struct)._fields_), struct


def _create(P, L, **kw):
    base = dict(n_seq=1, n_layer=1, n_kv=1, hpk=1, d=64, dv=64, m=8, w=16, sink=2, rect=0,
                exact_cap=0, ridge_rel=0.0)
    base.update(kw)
    cfg = P.o1_config(*[base[f] for f, _ in P.o1_config._fields_])
    h = ctypes.c_void_p()
    rc = L.o1_create_groups(ctypes.byref(cfg), ctypes.byref(h))
    return rc, h


@pytest.mark.parametrize("kw,code", [
    (dict(m=3), 1), (dict(w=0), 1), (dict(hpk=0), 1), (dict(sink=-1), 1), (dict(d=0), 1),
    (dict(dv=0), 1), (dict(n_seq=0), 1), (dict(n_layer=0), 1), (dict(n_kv=0), 1), (dict(rect=7), 1),
    (dict(d=72, dv=72), 6), (dict(d=512, dv=512), 6), (dict(hpk=65), 6),
    (dict(m=65), 6),
    (dict(d=64, dv=128), 6), (dict(d=96, dv=64), 6),
    (dict(d=192, dv=192), 6), (dict(d=128, dv=192), 6), (dict(d=192, dv=64), 6),
    (dict(hpk=5, w=596, sink=4), 6),  # run as 8 heads: 8 * 600 near logits pass 32 KB
    (dict(hpk=12, w=596, sink=4), 6),  # blocks of 8 and 4 heads: the 8-head block's logits pass 32 KB
    (dict(w=4095), 6), (dict(hpk=2, w=2040, sink=9), 6), (dict(exact_cap=-1), 1), (dict(n_seq=1 << 20, exact_cap=1 << 22), 1),
    (dict(ridge_rel=-1e-6), 1), (dict(ridge_rel=float("inf")), 1), (dict(ridge_rel=float("nan")), 1),
])
def test_create_rejects_before_touching_the_device(kw, code):
    P, L = _lib()
    rc, h = _create(P, L, **kw)
    assert rc == code, (kw, rc, P.o1_last_error())
    assert not h.value
    assert P.o1_last_error()


@pytest.mark.parametrize("kw", [
    dict(d=80, dv=80, hpk=5, w=1020, sink=4),     # blocks of 4 heads: 4 * 1024 near logits fit 32 KB
    dict(d=192, dv=128, hpk=64, m=32, w=128, sink=4),
    dict(d=256, dv=256, hpk=2, m=64, w=128, sink=4),
    dict(d=96, dv=96, hpk=13, m=64, w=256, sink=4),
    dict(d=128, dv=128, hpk=1, m=32, w=4092, sink=4),   # one head: 4096 near logits fit 32 KB
    dict(d=64, dv=64, hpk=2, m=32, w=2040, sink=8),
])
def test_create_passes_the_shape_checks_of_compiled_shapes(kw):
    # Without a GPU the creation fails later, at the device (O1_EHIP / O1_ENOMEM);
    # with one it succeeds.  Either way the shape checks let it through.
    P, L = _lib()
    rc, h = _create(P, L, **kw)
    if rc == 0:
        L.o1_destroy_groups(h)
    assert rc not in (P.O1_EINVAL, P.O1_EUNSUPPORTED), (kw, rc, P.o1_last_error())


def test_null_arguments_are_rejected():
    P, L = _lib()
    assert L.o1_create_groups(None, None) == P.O1_EINVAL
    assert L.o1_prefill(None, None, None, None, 300, None, None) == P.O1_EINVAL
    assert L.o1_step(None, None, None, None, None, None) == P.O1_EINVAL
    assert L.o1_prefill_layer(None, 0, None, 300, None, None) == P.O1_EINVAL
    assert L.o1_step_layer(None, 0, None, None, None, None, None) == P.O1_EINVAL
    info = P.o1_info()
    assert L.o1_get_info(None, ctypes.byref(info)) == P.O1_EINVAL
    n = ctypes.c_size_t()
    assert L.o1_field_bytes(None, 0, ctypes.byref(n)) == P.O1_EINVAL
    assert L.o1_read_field(None, 0, None, 0, None) == P.O1_EINVAL
    assert L.o1_write_field(None, 0, None, 0, None) == P.O1_EINVAL
    L.o1_destroy_groups(None)  # no-op
    assert "null" in P.o1_last_error()


def test_binding_refuses_host_tensors():
    import torch

    P, L = _lib()
    with pytest.raises((ValueError, TypeError)):
        P._dev_ptr(torch.zeros(4), "x", 4)


def test_exact_comparator_validation_without_device():
    P, L = _lib()
    n = ctypes.c_size_t()
    good = dict(n_groups=4, hpk=2, d=128, dv=128, cap=100, first=0, n_keys=100, scale=0.0)
    for kw, code in [(dict(first=100), 1), (dict(n_keys=101), 1), (dict(first=-1), 1),
                     (dict(n_groups=0), 1), (dict(hpk=65), 6), (dict(d=72, dv=72), 6),
                     (dict(dv=64), 6), (dict(d=192, dv=192), 6), (dict(d=128, dv=192), 6)]:
        args = {**good, **kw}
        desc = P.o1_exact_desc(*[args[f] for f, _ in P.o1_exact_desc._fields_])
        assert L.o1_exact_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)) == code, kw
    desc = P.o1_exact_desc(*[good[f] for f, _ in P.o1_exact_desc._fields_])
    assert L.o1_exact_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)) == 0
    assert n.value == 0  # 100 keys fit one chunk of one work-group: no partials
    # few groups and 1000 keys: the range splits over ceil(1000/128) = 8 work-groups,
    # each writing (max, sum, numerator[dv]) per head
    args = {**good, "cap": 1000, "n_keys": 1000}
    desc = P.o1_exact_desc(*[args[f] for f, _ in P.o1_exact_desc._fields_])
    assert L.o1_exact_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)) == 0
    assert n.value == 8 * (4 * 8 * 2 * (128 + 2))
    # keys of 192 floats with values of 128: the partials are dv wide
    desc = P.o1_exact_desc(*[{**args, "d": 192}[f] for f, _ in P.o1_exact_desc._fields_])
    assert L.o1_exact_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)) == 0
    assert n.value == 8 * (4 * 8 * 2 * (128 + 2))
    assert L.o1_exact_attend(ctypes.byref(desc), None, None, None, None, None, 0, None) == 1
    assert L.o1_exact_workspace_bytes(None, ctypes.byref(n)) == 1


def test_handle_released_during_a_capture_is_destroyed_later(monkeypatch):
    """A handle closed (or finalised by a garbage-collection pass) while the
    current stream is capturing a HIP graph is queued instead of freed, and
    destroyed at the next close or create outside a capture."""
    import ctypes

    import streaming_nystr_attention_amd as P

    destroyed = []
    monkeypatch.setattr(P, "o1_destroy_groups", lambda h: destroyed.append(h.value))
    capturing = [True]
    monkeypatch.setattr(P, "_capturing", lambda: capturing[0])
    grp = object.__new__(P.O1Groups)
    grp._h = ctypes.c_void_p(0x1234)
    grp.close()
    assert destroyed == [] and [h.value for h in P._DEFERRED_HANDLES] == [0x1234]
    grp.close()  # closing again neither frees nor queues twice
    assert destroyed == [] and len(P._DEFERRED_HANDLES) == 1
    capturing[0] = False
    other = object.__new__(P.O1Groups)
    other._h = ctypes.c_void_p(0x5678)
    other.close()
    assert destroyed == [0x5678, 0x1234] and P._DEFERRED_HANDLES == []


def test_exact_noalloc_refuses_launches_beyond_its_buffer_without_device():
    # 1020 groups of 8 heads over 4096 keys split in two: 1020 * 2 * 8 * (128 + 2)
    # doubles of partials, 16.9 MB, above the 16 MiB static buffer.  The check
    # comes before any device work (the tensors are never touched).
    P, L = _lib()
    desc = P.o1_exact_desc(1020, 8, 128, 128, 4096, 0, 4096, 0.0)
    n = ctypes.c_size_t()
    assert L.o1_exact_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)) == 0
    assert n.value > (16 << 20)
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced
    rc = L.o1_exact_attend_noalloc(ctypes.byref(desc), fake, fake, fake, fake, None)
    assert rc == P.O1_EINVAL
    assert "static buffer" in P.o1_last_error()
    assert L.o1_exact_attend_noalloc(None, fake, fake, fake, fake, None) == P.O1_EINVAL
    small = P.o1_exact_desc(4, 2, 128, 128, 100, 0, 100, 0.0)
    assert L.o1_exact_attend_noalloc(ctypes.byref(small), None, fake, fake, fake, None) == P.O1_EINVAL
