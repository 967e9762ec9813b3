"""Host-side checks of libmoe (no GPU needed): the library loads, exports every
entry point include/moe.h declares, and rejects bad arguments before enqueuing
anything (validation is synchronous and touches no device)."""
import ctypes
import os
import re

import pytest

import quantized_moe_ffn_amd as qm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "moe.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    lib = qm.load_library()
    declared = _declared()
    assert "moe_route_topk" in declared and "moe_expert_ffn_q" in declared and "moe_combine" in declared
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(qm.EXPORTS)


def test_abi_version():
    assert qm.moe_abi_version() == 1


def _routing_null():
    return qm.moe_routing(*(ctypes.c_void_p(8 * (i + 1)) for i in range(7)))


@pytest.mark.parametrize("T,E,k,msg", [
    (0, 8, 2, "T = 0"), (1, 0, 1, "E = 0"), (1, 2048, 2, "E = 2048"), (1, 8, 9, "k = 9"),
    (1, 64, 17, "k = 17"), (1, 8, 0, "k = 0"),
])
def test_route_rejects_bad_shapes(T, E, k, msg):
    lib = qm.load_library()
    r = _routing_null()
    st = lib.moe_route_topk(ctypes.c_void_p(256), T, E, k, 1, ctypes.byref(r), None, 0, None)
    assert st == 1
    assert msg in qm.moe_last_error()


def test_route_rejects_missing_workspace_for_large_batches():
    lib = qm.load_library()
    r = _routing_null()
    need = qm.moe_route_workspace_bytes(4096, 256, 8)
    assert need > 0
    st = lib.moe_route_topk(ctypes.c_void_p(256), 4096, 256, 8, 1, ctypes.byref(r), None, 0, None)
    assert st == 3 and "workspace" in qm.moe_last_error()


def test_quantize_rejects_bad_hidden():
    lib = qm.load_library()
    st = lib.moe_quantize_act(ctypes.c_void_p(256), 4, 300, ctypes.c_void_p(256), ctypes.c_void_p(256), None)
    assert st == 1 and "H = 300" in qm.moe_last_error()


def _qm(qt, rows, cols, E=4):
    rb = cols // qm.BLOCK_WEIGHTS[qt] * qm.BLOCK_BYTES[qt]
    return qm.moe_qmatrix(4096, qt, rows, cols, 0, rb, rb * rows)


def _layer(H=512, I=256, E=4, qd=qm.MOE_Q4_K):
    L = qm.moe_layer()
    L.n_experts, L.hidden, L.inter = E, H, I
    L.gate, L.up, L.down = _qm(qm.MOE_Q4_K, I, H, E), _qm(qm.MOE_Q4_K, I, H, E), _qm(qd, H, I, E)
    return L


def test_ffn_validation_messages():
    lib = qm.load_library()
    r = _routing_null()
    L = _layer()
    need = lib.moe_ffn_workspace_bytes(ctypes.byref(L), 2, 2, 1)
    assert need >= 2 * 2 * 256 * 4
    args = lambda L, ws=need: (ctypes.byref(L), ctypes.byref(r), 2, 2, ctypes.c_void_p(256), None, None, 1,
                               ctypes.c_void_p(256), None, ctypes.c_void_p(4096), ws, None)
    bad = _layer()
    bad.down.qtype = 3
    assert lib.moe_expert_ffn_q(*args(bad)) == 2 and "down.qtype = 3" in qm.moe_last_error()
    bad = _layer()
    bad.gate.row_bytes += 144
    assert lib.moe_expert_ffn_q(*args(bad)) == 1 and "gate.row_bytes" in qm.moe_last_error()
    bad = _layer(H=300)
    assert lib.moe_expert_ffn_q(*args(bad)) == 1 and "hidden = 300" in qm.moe_last_error()
    bad = _layer()
    bad.has_shared = 1
    bad.sh_gate, bad.sh_up, bad.sh_down = _qm(12, 256, 512, 1), _qm(12, 256, 512, 1), _qm(8, 512, 256, 1)
    assert lib.moe_expert_ffn_q(*args(bad)) in (1, 2)
    good = _layer()
    assert lib.moe_expert_ffn_q(*args(good, need - 1)) == 3 and "workspace" in qm.moe_last_error()
    # int8 path without xq/xd
    st = lib.moe_expert_ffn_q(ctypes.byref(good), ctypes.byref(r), 2, 2, None, None, None, 2,
                              ctypes.c_void_p(256), None, ctypes.c_void_p(4096), 1 << 20, None)
    assert st == 1 and "int8 path needs xq" in qm.moe_last_error()


def test_dequant_validation():
    lib = qm.load_library()
    assert lib.moe_dequant_q(ctypes.c_void_p(256), 12, 100, ctypes.c_void_p(256), None) == 1
    assert lib.moe_dequant_q(ctypes.c_void_p(257), 12, 256, ctypes.c_void_p(256), None) == 1
    assert lib.moe_dequant_q(ctypes.c_void_p(256), 2, 256, ctypes.c_void_p(256), None) == 2
    assert lib.moe_dequant_q(ctypes.c_void_p(256), 8, 0, ctypes.c_void_p(256), None) == 0
