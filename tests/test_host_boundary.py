"""The C-ABI boundary on the CPU: the library loads, exports every symbol
include/lso.h declares, the ctypes mirror matches the C layout, and the
host-side logic (validation, FP64-derived constants, workload shapes) is
right.  No device work is done here."""
import ctypes
import json
import math
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

import layer_streamed_optimizer_amd as lso
from layer_streamed_optimizer_amd import _native, configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lso.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lso_[a-z0-9_]+)\s*\(", text)) - {"lso_grad_fn"})


def test_library_exports_every_declared_symbol():
    lib = _native.lib()
    names = declared_functions()
    assert set(names) == set(_native.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _native._build.lib_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(lso_\w+)", out))
    assert set(names) <= exported


def test_struct_layout_matches_c_header():
    src = r"""
#include <stddef.h>
#include <stdio.h>
#include "lso.h"
#define F(T, f) printf("%s.%s %zu\n", #T, #f, offsetof(T, f));
int main(void) {
  printf("lso_block.size %zu\n", sizeof(lso_block));
  printf("lso_host_layer.size %zu\n", sizeof(lso_host_layer));
  F(lso_block, base) F(lso_block, n) F(lso_block, off_master) F(lso_block, off_m)
  F(lso_block, off_v) F(lso_block, off_grad) F(lso_block, off_weight) F(lso_block, grad_dtype)
  F(lso_block, weight_dtype) F(lso_block, opt) F(lso_block, layout) F(lso_block, t)
  F(lso_block, lr) F(lso_block, beta1) F(lso_block, beta2) F(lso_block, eps)
  F(lso_host_layer, host_base) F(lso_host_layer, bytes) F(lso_host_layer, n)
  F(lso_host_layer, off_master) F(lso_host_layer, off_m) F(lso_host_layer, off_v)
  F(lso_host_layer, dev_weight) F(lso_host_layer, opt) F(lso_host_layer, layout)
  F(lso_host_layer, t) F(lso_host_layer, lr) F(lso_host_layer, beta1) F(lso_host_layer, beta2)
  F(lso_host_layer, eps) F(lso_host_layer, sq_norm) F(lso_host_layer, grad_dtype)
  F(lso_host_layer, reserved)
  printf("lso_file_layer.size %zu\n", sizeof(lso_file_layer));
  F(lso_file_layer, fd) F(lso_file_layer, flags) F(lso_file_layer, file_offset)
  F(lso_file_layer, bytes) F(lso_file_layer, n) F(lso_file_layer, off_master)
  F(lso_file_layer, off_m) F(lso_file_layer, off_v) F(lso_file_layer, dev_weight)
  F(lso_file_layer, opt) F(lso_file_layer, layout) F(lso_file_layer, t) F(lso_file_layer, lr)
  F(lso_file_layer, beta1) F(lso_file_layer, beta2) F(lso_file_layer, eps) F(lso_file_layer, sq_norm)
  F(lso_file_layer, grad_dtype) F(lso_file_layer, reserved)
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "l.c")
        exe = os.path.join(d, "l")
        open(c, "w").write(src)
        subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe])
        lines = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    got = dict(l.split() for l in lines if l)
    assert int(got["lso_block.size"]) == ctypes.sizeof(_native.LsoBlock) == lso.BLOCK_DTYPE.itemsize
    assert int(got["lso_host_layer.size"]) == ctypes.sizeof(_native.LsoHostLayer)
    assert int(got["lso_file_layer.size"]) == ctypes.sizeof(_native.LsoFileLayer)
    for struct, cls in (("lso_block", _native.LsoBlock), ("lso_host_layer", _native.LsoHostLayer),
                        ("lso_file_layer", _native.LsoFileLayer)):
        for fname, _ in cls._fields_:
            assert int(got[f"{struct}.{fname}"]) == getattr(cls, fname).offset, (struct, fname)


def test_header_constants_match_binding():
    text = open(HEADER).read()
    defs = dict(re.findall(r"#define\s+(LSO_[A-Z0-9_]+)\s+(\d+)u?\b", text))
    for name in ("LSO_COPY_SDMA_PAIR", "LSO_COPY_DMA_IN", "LSO_COPY_KERNELS", "LSO_COPY_DMA",
                 "LSO_FILE_SYNC", "LSO_FILE_SHADOW", "LSO_SHADOW_HEADER_BYTES", "LSO_TILE_ELEMS",
                 "LSO_NOALLOC_MAX_BLOCKS"):
        assert int(defs[name]) == getattr(_native, name), name
    codes = [getattr(_native, n) for n in ("LSO_COPY_SDMA_PAIR", "LSO_COPY_DMA_IN", "LSO_COPY_KERNELS",
                                           "LSO_COPY_DMA")]
    assert sorted(codes) == sorted(_native.COPY_MODE_NAMES)


def test_copy_mode_of_no_context():
    assert _native.lib().lso_stream_copy_mode(None, None, None) == -1


def test_status_strings():
    lib = _native.lib()
    for s in range(8):
        assert lib.lso_status_string(s)
    assert lib.lso_status_string(99) == b"unknown status"


# ---------------------------------------------------------------- validation

A = 1 << 32   # fake device addresses: validation never touches memory


def table(rows):
    return lso.BlockTable.from_rows(rows)


def row(k=0, n=1000, **kw):
    base = A + k * (1 << 24)
    r = dict(n=n, master=base, m=base + (1 << 20), v=base + (2 << 20), grad=base + (3 << 20),
             weight=base + (4 << 20))
    r.update(kw)
    return r


def test_valid_tables_pass():
    assert lso.validate(table([row(0), row(1), row(2, opt=lso.LSO_OPT_SGD)])) == 0
    assert lso.validate(table([])) == 0
    assert lso.validate(table([row(0, n=0, master=A + 4)])) == 0   # n == 0: no-op block


@pytest.mark.parametrize("field", ["master", "m", "v", "grad", "weight"])
def test_misaligned_array_is_rejected(field):
    r = row(0)
    r[field] = r[field] + 8
    assert lso.validate(table([r])) == _native.LSO_E_ALIGN
    assert field in lso.last_error()


def test_sgd_ignores_moment_pointers():
    r = row(0, opt=lso.LSO_OPT_SGD, m=A + 3, v=0)
    assert lso.validate(table([r])) == 0


def test_overlap_within_and_across_blocks():
    r = row(0)
    r["v"] = r["m"] + 16           # v overlaps m
    assert lso.validate(table([r])) == _native.LSO_E_OVERLAP
    a, b = row(0), row(1)
    b["master"] = a["weight"]      # written arrays of two blocks collide
    assert lso.validate(table([a, b])) == _native.LSO_E_OVERLAP
    a, b = row(0), row(1)
    b["grad"] = a["grad"]          # gradients may alias (read-only)
    assert lso.validate(table([a, b])) == 0
    a, b = row(0), row(1)
    b["grad"] = a["master"]        # a read array under a written one
    assert lso.validate(table([a, b])) == _native.LSO_E_OVERLAP


def test_adjacent_arrays_do_not_overlap():
    n = 1024
    r = dict(n=n, master=A, m=A + 4 * n, v=A + 8 * n, grad=A + 12 * n, weight=A + 14 * n)
    assert lso.validate(table([r])) == 0
    r["weight"] -= 16
    assert lso.validate(table([r])) == _native.LSO_E_OVERLAP


@pytest.mark.parametrize("kw,code", [
    (dict(t=0), _native.LSO_E_INVALID),
    (dict(beta1=1.0), _native.LSO_E_INVALID),
    (dict(beta2=-0.1), _native.LSO_E_INVALID),
    (dict(eps=-1e-8), _native.LSO_E_INVALID),
    (dict(eps=float("inf")), _native.LSO_E_INVALID),
    (dict(lr=float("nan")), _native.LSO_E_INVALID),
    (dict(opt=7), _native.LSO_E_DTYPE),
])
def test_bad_hyper_parameters(kw, code):
    assert lso.validate(table([row(0, **kw)])) == code


def test_bad_dtype_and_layout():
    t = table([row(0)])
    t.arr[0]["grad_dtype"] = lso.LSO_DT_NONE
    assert lso.validate(t) == _native.LSO_E_DTYPE
    t = table([row(0)])
    t.arr[0]["weight_dtype"] = lso.LSO_DT_F32
    assert lso.validate(t) == _native.LSO_E_DTYPE
    t = table([row(0)])
    t.arr[0]["layout"] = 7
    assert lso.validate(t) == _native.LSO_E_INVALID
    t = table([row(0, opt=lso.LSO_OPT_SGD, layout=lso.LSO_LAYOUT_TILED)])
    assert lso.validate(t) == _native.LSO_E_DTYPE
    t = table([row(0, master=0)])
    assert lso.validate(t) == _native.LSO_E_INVALID


def test_fp32_gradients_span_four_bytes_per_element():
    """An FP32 gradient array covers 4n bytes: the same placement that is
    fine for BF16 gradients overlaps the next array with FP32 ones."""
    n = 1024
    r = dict(n=n, master=A, m=A + 4 * n, v=A + 8 * n, grad=A + 12 * n, weight=A + 14 * n)
    assert lso.validate(table([r])) == 0
    assert lso.validate(table([dict(r, grad_dtype=lso.LSO_DT_F32)])) == _native.LSO_E_OVERLAP
    r["weight"] = A + 16 * n
    assert lso.validate(table([dict(r, grad_dtype=lso.LSO_DT_F32)])) == 0
    tiled = lso.tiled_state_bytes(n)
    t = dict(n=n, master=A, grad=A + tiled, weight=A + tiled + 4 * n, layout=lso.LSO_LAYOUT_TILED)
    assert lso.validate(table([dict(t, grad_dtype=lso.LSO_DT_F32)])) == 0
    assert lso.validate(table([dict(t, grad_dtype=lso.LSO_DT_F32, weight=A + tiled + 2 * n)])) \
        == _native.LSO_E_OVERLAP
    assert lso.validate(table([dict(r, grad_dtype=lso.LSO_DT_F32, opt=lso.LSO_OPT_SGD)])) == 0
    # BF16 and FP32 gradient blocks in one call
    assert lso.validate(table([row(0, grad_dtype=lso.LSO_DT_F32), row(1)])) == 0


def test_adam_step_rejects_before_touching_the_device():
    """An invalid table returns its error without any HIP call, so this runs
    on a machine with no GPU."""
    r = row(0)
    r["master"] += 4
    with pytest.raises(lso.LsoError) as e:
        lso.adam_step(table([r]), stream=0)
    assert e.value.status == _native.LSO_E_ALIGN


def test_empty_adam_step_is_a_no_op():
    lso.adam_step(table([]), stream=0)
    lso.adam_step_noalloc(table([]), stream=0)


def test_noalloc_rejects_tables_beyond_its_scratch_before_touching_the_device():
    """lso_adam_step_noalloc: a call whose launches need more table entries
    than the fixed scratch array holds is refused with a clear error before
    any HIP call (this runs without a GPU); so are the usual invalid tables."""
    rows = [row(k, n=16) for k in range(_native.LSO_NOALLOC_MAX_BLOCKS + 1)]
    with pytest.raises(lso.LsoError) as e:
        lso.adam_step_noalloc(table(rows), stream=0)
    assert e.value.status == _native.LSO_E_INVALID and "exceed" in str(e.value)
    r = row(0)
    r["master"] += 4
    with pytest.raises(lso.LsoError) as e:
        lso.adam_step_noalloc(table([r]), stream=0)
    assert e.value.status == _native.LSO_E_ALIGN
    with pytest.raises(lso.LsoError) as e:
        lso.adam_step_noalloc(table([row(0), row(0)] + [row(k) for k in range(2, 7)]), stream=0)
    assert e.value.status == _native.LSO_E_OVERLAP


# ----------------------------------------------------------------- constants

def test_constants_are_fp64_rounded_once():
    for t in (1, 2, 10, 100, 10000):
        c = lso.block_constants(t=t, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
        f = np.float32
        expect = [f(0.9), f(0.1), f(0.999), f(1 - 0.999),
                  f(1e-3 / (1 - 0.9 ** t)), f(1 / math.sqrt(1 - 0.999 ** t)), f(1e-8), f(0)]
        assert np.array_equal(c, np.array(expect, np.float32)), t
    # the FP32 route the host must not take: 1 - fl32(0.999) is 1.3e-5 off
    assert abs(float(np.float32(1) - np.float32(0.999)) / (1 - 0.999) - 1) > 1e-5
    c = lso.block_constants(t=1, opt=lso.LSO_OPT_SGD, lr=0.015)
    assert c[4] == np.float32(0.015) and not c[:4].any()


def test_constants_reject_t0():
    with pytest.raises(lso.LsoError):
        lso.block_constants(t=0)


# -------------------------------------------------------------------- shapes

def test_workload_parameter_counts_match_the_pages():
    gold = json.load(open(os.path.join(GOLDEN, "state_accounting.json")))
    c3 = configs.get("c3")
    assert c3.params == gold["llama7b"]["params"] == 6_738_415_616
    assert abs(c3.params * 16 / 1e9 - gold["llama7b"]["state_GB"]) < 0.05
    assert configs.layer_params(**configs.LLAMA7B) == 202_383_360
    c2 = configs.get("c2")
    assert len(c2.blocks) == 308
    assert c2.params == 6_307_840
    assert abs(c2.params * 4 / 1e6 - gold["tinyllama_lora"]["adapter_MB"]) < 0.005
    assert abs(c2.params * 8 / 1e6 - gold["tinyllama_lora"]["adam_MB"]) < 0.01
    sizes = sorted({b.n for b in c2.blocks})
    assert sizes == [2048, 16384, 45056]
    assert sorted(b.n for b in c2.blocks[:14]) == [2048] * 2 + [16384] * 9 + [45056] * 3
    c1 = configs.get("c1")
    assert configs.layer_params(**configs.TINYLLAMA) == 44_044_288
    assert c1.params == 1_100_048_384
    assert round(c1.params / 1e9, 2) == gold["tinyllama_lora"]["base_params_billion"]
    c4 = configs.get("c4")
    assert configs.layer_params(**configs.LLAMA70B) == 855_654_400
    assert c4.params == 13_690_470_400
    assert configs.get("c0").params == 1 << 20


def test_resident_layout_is_page_aligned_and_disjoint():
    lay = configs.ResidentLayout([1000, 4096, 3, 65537])
    for offs in (lay.off_master, lay.off_m, lay.off_v, lay.off_grad, lay.off_weight):
        assert all(o % configs.PAGE == 0 for o in offs)
    spans = []
    for i, n in enumerate(lay.sizes):
        spans += [(lay.off_master[i], 4 * n), (lay.off_m[i], 4 * n), (lay.off_v[i], 4 * n)]
    spans.sort()
    for (a, la), (b, _) in zip(spans, spans[1:]):
        assert a + la <= b
    assert spans[-1][0] + spans[-1][1] <= lay.state_bytes
    off = configs.host_layer_layout(855_654_400)
    assert off[3] == 3 * configs.align(4 * 855_654_400) and off[3] % 4096 == 0


@pytest.mark.parametrize("tiled", [False, True])
def test_block_arena_is_page_aligned_disjoint_and_block_by_block(tiled):
    sizes = [1000, 4096, 3, 65537, 8193]
    a = configs.BlockArena(sizes, tiled=tiled, grad_sets=3)
    spans = []
    for b, n in enumerate(sizes):
        st = configs.tiled_state_bytes(n) if tiled else 4 * n
        if tiled:
            assert a.off_m[b] == a.off_v[b] == a.off_master[b]
            spans.append((a.off_master[b], st))
        else:
            spans += [(a.off_master[b], st), (a.off_m[b], st), (a.off_v[b], st)]
        spans.append((a.off_weight[b], 2 * n))
        spans += [(a.off_grad[r][b], 2 * n) for r in range(3)]
        # a block's arrays lie between its state and the next block's state
        nxt = a.off_master[b + 1] if b + 1 < len(sizes) else a.total_bytes
        assert a.off_master[b] < a.off_weight[b] < a.off_grad[0][b] < a.off_grad[2][b] < nxt
    for o, _ in spans:
        assert o % configs.PAGE == 0
    spans.sort()
    for (x, lx), (y, _) in zip(spans, spans[1:]):
        assert x + lx <= y
    assert spans[-1][0] + spans[-1][1] <= a.total_bytes
    one = configs.ResidentLayout(sizes, tiled=tiled)
    assert (a.state_bytes, a.grad_bytes, a.weight_bytes) == (one.state_bytes, one.grad_bytes, one.weight_bytes)
    assert a.total_bytes == a.state_bytes + a.weight_bytes + 3 * a.grad_bytes
    with pytest.raises(ValueError):
        configs.BlockArena(sizes, grad_sets=0)


def test_tiled_state_region_validation():
    n = 3 * 8192 + 5
    rb = lso.tiled_state_bytes(n)
    assert rb == 12 * 8192 * 4 == configs.tiled_state_bytes(n)
    assert lso.tiled_state_bytes(0) == 0 and lso.tiled_state_bytes(1) == 12 * 8192
    base = A
    ok = dict(n=n, master=base, m=None, v=None, grad=base + rb, weight=base + rb + 65536,
              layout=lso.LSO_LAYOUT_TILED)
    assert lso.validate(table([ok])) == 0
    # m / v are ignored for tiled blocks (they may be anything)
    assert lso.validate(table([dict(ok, m=A + 3, v=A + 5)])) == 0
    # the whole padded region counts: a gradient inside the padding overlaps
    bad = dict(ok, grad=base + 12 * 8192 * 3 + 4096)
    assert lso.validate(table([bad])) == _native.LSO_E_OVERLAP
    assert lso.validate(table([dict(ok, master=base + 8)])) == _native.LSO_E_ALIGN


def test_resident_layout_tiled():
    lay = configs.ResidentLayout([100, 8192, 8193], tiled=True)
    assert lay.off_master == lay.off_m == lay.off_v
    assert lay.off_master[1] - lay.off_master[0] == configs.align(configs.tiled_state_bytes(100))
    assert lay.state_bytes == sum(configs.align(configs.tiled_state_bytes(n)) for n in lay.sizes)
    assert configs.host_layer_layout(8193, tiled=True) == (0, 0, 0, configs.align(12 * 8192 * 2))


def test_norm_workspace_bytes_follow_the_launch_plan():
    """One FP64 per wave (4 per chunk): planar chunks of 1024 elements in
    calls under 32M planar elements, 4096 above; tiled chunks are an eighth
    of a state tile (1024 elements)."""
    per = 4 * 8
    assert lso.norm_workspace_bytes(table([])) == 0
    assert lso.norm_workspace_bytes(table([row(0, n=1), row(1, n=1024), row(2, n=1025)])) == per * (1 + 1 + 2)
    big = row(0, n=32 << 20)
    assert lso.norm_workspace_bytes(table([big])) == per * ((32 << 20) // 4096)
    t = dict(n=8193, master=A, grad=A + (1 << 20), layout=lso.LSO_LAYOUT_TILED)
    assert lso.norm_workspace_bytes(table([t, row(1, n=5000)])) == per * (9 + 5)


def _norms_status(tab, sq, ws, ws_bytes):
    return _native.lib().lso_adam_step_norms(tab.ptr, len(tab), sq, ws, ws_bytes, 0)


def test_norm_call_rejects_bad_buffers_before_touching_the_device():
    """Every case below is invalid, so nothing is enqueued (fake addresses)."""
    tab = table([row(0), row(1)])
    need = lso.norm_workspace_bytes(tab)
    sq, ws = A + (200 << 20), A + (300 << 20)
    E = _native
    assert _norms_status(tab, 0, ws, need) == E.LSO_E_INVALID
    assert _norms_status(tab, sq, 0, need) == E.LSO_E_INVALID
    assert _norms_status(tab, sq, ws, need - 8) == E.LSO_E_INVALID
    assert "workspace" in lso.last_error()
    assert _norms_status(tab, sq + 4, ws, need) == E.LSO_E_ALIGN
    assert _norms_status(tab, row(0)["master"] + 16, ws, need) == E.LSO_E_OVERLAP
    assert _norms_status(tab, sq, row(1)["grad"], need) == E.LSO_E_OVERLAP
    assert _norms_status(tab, sq, sq, need) == E.LSO_E_OVERLAP
    bad = table([row(0), row(1, beta1=1.5)])
    assert _norms_status(bad, sq, ws, need) == E.LSO_E_INVALID
