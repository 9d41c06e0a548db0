"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and rejects invalid arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import routing_dispatch_expert_moe_amd as M
from routing_dispatch_expert_moe_amd import _lib as L
from oracle import moe_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from routing_dispatch_expert_moe_amd import build
        build.build()
    return M.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_path():
    names = declared_functions()
    for n in ("moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_router_logits",
              "moe_pack_weights", "moe_check_error", "moe_ffn_up", "moe_ffn_down",
              "moe_forward_fused", "moe_quantize_fp8", "moe_expert_ffn_fp8", "moe_ffn_up_fp8",
              "moe_ffn_down_fp8", "moe_expert_ffn_list", "moe_ffn_up_list", "moe_ffn_down_list",
              "moe_route_reroute", "moe_forward_fused_reroute", "moe_forward_fused_fp8",
              "moe_set_fused_overlap", "moe_forward_fused_list", "moe_expert_ffn_fp8_list",
              "moe_ffn_up_fp8_list", "moe_ffn_down_fp8_list", "moe_forward_fused_fp8_list"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(L.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name
        assert name in L.SIGNATURES, f"binding lacks {name}"


def test_status_strings(lib):
    for s in range(7):
        assert lib.moe_status_string(s).decode().startswith("MOE_")
    assert b"unknown" in lib.moe_status_string(99)


def test_capacity_matches_oracle_rule(lib):
    for T, k, E, cf in [(16384, 2, 128, 1.25), (32 * 2048, 2, 128, 1.0), (100, 2, 8, 0.1),
                        (30, 1, 10, 0.3), (7, 3, 5, 2.0), (1, 1, 1, 1.0), (0, 2, 4, 1.0)]:
        assert M.moe_capacity(T, k, E, cf) == O.capacity(T, k, E, cf)
    assert M.moe_capacity(10, 1, 1, None) == -1


def test_max_rows_and_workspace(lib):
    assert M.moe_max_rows(16384, 2, 32, 320) == 32 * 320
    assert M.moe_max_rows(128, 8, 256, -1) == 1024
    assert M.moe_max_rows(10, 2, 4, 100) == 20
    assert M.moe_workspace_bytes(4096, 8, 2, 8) >= 256 + 2 * 16 * 8 * 4
    assert M.moe_workspace_bytes(10, 8, 9, 8) == 0      # k > MOE_MAX_K
    assert M.moe_workspace_bytes(10, 8, 2, 9) == 0      # E_loc > E


FAKE = 4096      # aligned, never dereferenced: every call below fails validation first
MIS = 4098       # not 16-byte aligned


def test_route_validation(lib):
    r = lib.moe_route
    assert r(FAKE, 10, 8, 0, 0, FAKE, FAKE, None) == L.MOE_ERR_INVALID_TOPK
    assert r(FAKE, 10, 8, 9, 0, FAKE, FAKE, None) == L.MOE_ERR_INVALID_TOPK
    assert r(FAKE, 10, 4, 5, 0, FAKE, FAKE, None) == L.MOE_ERR_INVALID_TOPK
    assert r(FAKE, 10, 2000, 2, 0, FAKE, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert r(FAKE, 10, 8, 2, 7, FAKE, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert r(None, 10, 8, 2, 0, FAKE, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert r(MIS, 10, 8, 2, 0, FAKE, FAKE, None) == L.MOE_ERR_MISALIGNED
    assert r(FAKE, -1, 8, 2, 0, FAKE, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert r(None, 0, 8, 2, 0, None, None, None) == L.MOE_OK   # empty batch: nothing to do


def test_dispatch_validation(lib):
    d = lib.moe_dispatch
    ok = dict(idx=FAKE, T=10, E=8, k=2, cap=-1, e0=0, e1=8, x=FAKE, d=64, dt=L.MOE_BF16,
              counts=FAKE, off=FAKE, sp=FAKE, pp=FAKE, nk=FAKE, xp=FAKE, ws=FAKE, wsb=0)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return d(a["idx"], a["T"], a["E"], a["k"], a["cap"], a["e0"], a["e1"], a["x"], a["d"],
                 a["dt"], a["counts"], a["off"], a["sp"], a["pp"], a["nk"], a["xp"], a["ws"],
                 a["wsb"], None)

    assert call() == L.MOE_ERR_WORKSPACE
    assert call(wsb=2047) == L.MOE_ERR_WORKSPACE    # smaller than the 2 KiB header
    assert call(k=9) == L.MOE_ERR_INVALID_TOPK
    assert call(e0=3, e1=3) == L.MOE_ERR_INVALID_ARG
    assert call(e1=9) == L.MOE_ERR_INVALID_ARG
    assert call(d=12) == L.MOE_ERR_UNSUPPORTED      # bf16 rows of 24 bytes
    assert call(dt=5) == L.MOE_ERR_UNSUPPORTED
    assert call(xp=None) == L.MOE_ERR_INVALID_ARG
    assert call(pp=MIS) == L.MOE_ERR_MISALIGNED
    assert call(ws=None) == L.MOE_ERR_INVALID_ARG


def test_ffn_validation(lib):
    f = lib.moe_expert_ffn
    args = [FAKE, FAKE, 8, 100, 4096, 14336, L.MOE_BF16, FAKE, FAKE, FAKE, FAKE, None, 0, None]
    bad_d = list(args); bad_d[4] = 4000
    assert f(*bad_d) == L.MOE_ERR_UNSUPPORTED
    bad_e = list(args); bad_e[2] = 0
    assert f(*bad_e) == L.MOE_ERR_INVALID_ARG
    mis = list(args); mis[7] = MIS
    assert f(*mis) == L.MOE_ERR_MISALIGNED
    nul = list(args); nul[1] = None
    assert f(*nul) == L.MOE_ERR_INVALID_ARG
    f32 = list(args); f32[6] = L.MOE_F32; f32[4] = 6
    assert f(*f32) == L.MOE_ERR_UNSUPPORTED
    up = lib.moe_ffn_up
    assert up(FAKE, FAKE, 8, -1, 64, 64, L.MOE_BF16, FAKE, FAKE, None, 0, None) == L.MOE_ERR_INVALID_ARG


def test_reroute_validation(lib):
    r = lib.moe_route_reroute
    need = lib.moe_workspace_bytes(100, 8, 2, 8)
    ok = [FAKE, 100, 8, 2, 0, 30, FAKE, FAKE, FAKE, need, None]
    bad = list(ok); bad[3] = 9
    assert r(*bad) == L.MOE_ERR_INVALID_TOPK
    bad = list(ok); bad[4] = 3             # gate
    assert r(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(ok); bad[5] = -2            # capacity
    assert r(*bad) == L.MOE_ERR_INVALID_ARG
    # the fused launch's readiness counters (E_loc words, one 256-byte block
    # here) follow the rerouting scratch: one byte short of that scratch fails
    bad = list(ok); bad[9] = need - 256 - 1
    assert r(*bad) == L.MOE_ERR_WORKSPACE
    bad = list(ok); bad[8] = None
    assert r(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(ok); bad[0] = MIS
    assert r(*bad) == L.MOE_ERR_MISALIGNED
    assert r(None, 0, 8, 2, 0, 30, None, None, None, 0, None) == L.MOE_OK   # empty batch
    # the workspace holds the k + 1 candidates per token beyond the dispatch scratch
    assert lib.moe_workspace_bytes(1000, 8, 8, 8) - lib.moe_workspace_bytes(1000, 8, 1, 8) >= 1000 * 7 * 8 - 512
    # and one readiness word per local expert, in 256-byte blocks
    assert lib.moe_workspace_bytes(1000, 256, 8, 256) - lib.moe_workspace_bytes(1000, 256, 8, 1) == 1024 - 256


def test_fused_overlap_setting(lib):
    # host-only: the setting is validated and stored, no GPU call
    for mode in (L.MOE_OVERLAP_NEVER, L.MOE_OVERLAP_ALWAYS, L.MOE_OVERLAP_AUTO):
        assert lib.moe_set_fused_overlap(mode) == L.MOE_OK
    assert lib.moe_set_fused_overlap(3) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_set_fused_overlap(-1) == L.MOE_ERR_INVALID_ARG
    M.moe_set_fused_overlap("auto")


def test_list_validation(lib):
    f = lib.moe_expert_ffn_list
    ok = [FAKE, FAKE, 8, 100, 4096, 1024, L.MOE_BF16, FAKE, FAKE, FAKE, FAKE, None]
    bad = list(ok); bad[7] = None          # no w13 table
    assert f(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(ok); bad[8] = MIS           # misaligned w2 table
    assert f(*bad) == L.MOE_ERR_MISALIGNED
    bad = list(ok); bad[4] = 100           # bf16 d % 64
    assert f(*bad) == L.MOE_ERR_UNSUPPORTED
    bad = list(ok); bad[6] = 9             # dtype
    assert f(*bad) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_ffn_up_list(FAKE, FAKE, 0, 100, 64, 64, L.MOE_BF16, FAKE, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_ffn_down_list(FAKE, FAKE, 8, 100, 64, 64, L.MOE_BF16, None, FAKE, None) == L.MOE_ERR_INVALID_ARG


def test_fp8_validation(lib):
    qz = lib.moe_quantize_fp8
    assert qz(None, 1, 128, 128, FAKE, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert qz(FAKE, 0, 128, 128, FAKE, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert qz(FAKE, 1, 100, 128, FAKE, FAKE, None) == L.MOE_ERR_UNSUPPORTED   # rows % 128
    assert qz(FAKE, 1, 128, 192, FAKE, FAKE, None) == L.MOE_ERR_UNSUPPORTED   # K % 128
    assert qz(FAKE, 1, 128, 128, MIS, FAKE, None) == L.MOE_ERR_MISALIGNED
    f = lib.moe_expert_ffn_fp8
    ok = [FAKE, FAKE, 8, 100, 4096, 1024, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None]
    bad = list(ok); bad[5] = 1000          # f % 64
    assert f(*bad) == L.MOE_ERR_UNSUPPORTED
    bad = list(ok); bad[5] = 960           # f % 128 (bf16 alone would take it)
    assert f(*bad) == L.MOE_ERR_UNSUPPORTED
    bad = list(ok); bad[7] = None          # no scales
    assert f(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(ok); bad[9] = MIS
    assert f(*bad) == L.MOE_ERR_MISALIGNED
    bad = list(ok); bad[2] = 0
    assert f(*bad) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_ffn_up_fp8(FAKE, FAKE, 8, 100, 4096, 1024, FAKE, None, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_ffn_down_fp8(FAKE, FAKE, 8, 100, 4096, 1024, FAKE, MIS, FAKE, None) == L.MOE_ERR_MISALIGNED
    # the TensorList form: the tables stand where the codes and scales do
    fl = lib.moe_expert_ffn_fp8_list
    for i, code in ((6, L.MOE_ERR_INVALID_ARG), (7, L.MOE_ERR_INVALID_ARG),
                    (8, L.MOE_ERR_INVALID_ARG), (9, L.MOE_ERR_INVALID_ARG)):
        bad = list(ok); bad[i] = None          # a missing code or scale table
        assert fl(*bad) == code
    bad = list(ok); bad[8] = MIS
    assert fl(*bad) == L.MOE_ERR_MISALIGNED
    bad = list(ok); bad[5] = 960
    assert fl(*bad) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_ffn_up_fp8_list(FAKE, FAKE, 8, 100, 4096, 1024, FAKE, None, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_ffn_down_fp8_list(FAKE, FAKE, 8, 100, 4096, 1024, MIS, FAKE, FAKE, None) == L.MOE_ERR_MISALIGNED
    assert lib.moe_ffn_down_fp8_list(FAKE, FAKE, 0, 100, 4096, 1024, FAKE, FAKE, FAKE, None) == L.MOE_ERR_INVALID_ARG


def test_combine_router_pack_validation(lib):
    assert lib.moe_combine(FAKE, FAKE, FAKE, 10, 9, 64, L.MOE_BF16, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(FAKE, FAKE, FAKE, 10, 2, 6, L.MOE_F32, FAKE, None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_combine(FAKE, FAKE, MIS, 10, 2, 64, L.MOE_BF16, FAKE, None) == L.MOE_ERR_MISALIGNED
    assert lib.moe_router_logits(FAKE, FAKE, 10, 4096, L.MOE_MAX_E + 1, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_router_logits(FAKE, FAKE, 10, 4092, 8, FAKE, None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_pack_weights(FAKE, FAKE, FAKE, 0, 64, 64, L.MOE_BF16, FAKE, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_pack_weights(FAKE, MIS, FAKE, 2, 64, 64, L.MOE_BF16, FAKE, FAKE, None) == L.MOE_ERR_MISALIGNED
    assert lib.moe_check_error(None, None) == L.MOE_ERR_INVALID_ARG


def test_fused_validation(lib):
    f = lib.moe_forward_fused
    ws_ok = M.moe_workspace_bytes(100, 8, 2, 8)
    ok = dict(lg=FAKE, x=FAKE, T=100, E=8, k=2, gate=0, cap=-1, e0=0, e1=8, d=128, f=256,
              dt=L.MOE_BF16, w13=FAKE, w2=FAKE, idx=FAKE, w=FAKE, counts=FAKE, off=FAKE, sp=FAKE,
              pp=FAKE, nk=FAKE, h=FAKE, yp=FAKE, y=FAKE, ws=FAKE, wsb=ws_ok)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["lg"], a["x"], a["T"], a["E"], a["k"], a["gate"], a["cap"], a["e0"], a["e1"],
                 a["d"], a["f"], a["dt"], a["w13"], a["w2"], a["idx"], a["w"], a["counts"],
                 a["off"], a["sp"], a["pp"], a["nk"], a["h"], a["yp"], a["y"], a["ws"], a["wsb"],
                 None)

    assert call(k=9) == L.MOE_ERR_INVALID_TOPK
    assert call(k=0) == L.MOE_ERR_INVALID_TOPK
    assert call(E=2000) == L.MOE_ERR_INVALID_ARG
    assert call(gate=5) == L.MOE_ERR_INVALID_ARG
    assert call(e0=4, e1=2) == L.MOE_ERR_INVALID_ARG
    assert call(T=-1) == L.MOE_ERR_INVALID_ARG
    assert call(d=100) == L.MOE_ERR_UNSUPPORTED         # bf16 needs d % 64 == 0
    assert call(dt=7) == L.MOE_ERR_UNSUPPORTED
    assert call(x=None) == L.MOE_ERR_INVALID_ARG
    assert call(ws=None) == L.MOE_ERR_INVALID_ARG
    assert call(y=MIS) == L.MOE_ERR_MISALIGNED
    assert call(h=MIS) == L.MOE_ERR_MISALIGNED
    assert call(wsb=2047) == L.MOE_ERR_WORKSPACE
    # bf16 operands beyond 32-bit byte offsets are refused up front
    assert call(T=600000, k=8, E=8, d=4096, f=4096) == L.MOE_ERR_UNSUPPORTED
    # the rerouting form takes the same arguments and needs the rerouting scratch too
    g = lib.moe_forward_fused_reroute

    def call_r(**kw):
        a = dict(ok)
        a.update(kw)
        return g(a["lg"], a["x"], a["T"], a["E"], a["k"], a["gate"], a["cap"], a["e0"], a["e1"],
                 a["d"], a["f"], a["dt"], a["w13"], a["w2"], a["idx"], a["w"], a["counts"],
                 a["off"], a["sp"], a["pp"], a["nk"], a["h"], a["yp"], a["y"], a["ws"], a["wsb"],
                 None)

    # FP8 weights: scales required, d and f multiples of 128 and at least 256
    h8 = lib.moe_forward_fused_fp8

    def call_8(**kw):
        a = dict(ok, d=256, f=512, s13=FAKE, s2=FAKE)
        a.update(kw)
        return h8(a["lg"], a["x"], a["T"], a["E"], a["k"], a["gate"], a["cap"], a["e0"], a["e1"],
                  a["d"], a["f"], a["w13"], a["s13"], a["w2"], a["s2"], a["idx"], a["w"],
                  a["counts"], a["off"], a["sp"], a["pp"], a["nk"], a["h"], a["yp"], a["y"],
                  a["ws"], a["wsb"], None)

    assert call_8(s13=None) == L.MOE_ERR_INVALID_ARG
    assert call_8(s2=None) == L.MOE_ERR_INVALID_ARG
    assert call_8(d=192) == L.MOE_ERR_UNSUPPORTED        # not a multiple of the 128 scale block
    assert call_8(d=128) == L.MOE_ERR_UNSUPPORTED        # below the pipeline's depth (256)
    assert call_8(f=128) == L.MOE_ERR_UNSUPPORTED
    assert call_8(k=9) == L.MOE_ERR_INVALID_TOPK
    assert call_8(s13=MIS) == L.MOE_ERR_MISALIGNED
    assert call_8(wsb=2047) == L.MOE_ERR_WORKSPACE
    # the fused FP8 layer on per-expert tables: the same checks on the tables
    h8l = lib.moe_forward_fused_fp8_list

    def call_8l(**kw):
        a = dict(ok, d=256, f=512, s13=FAKE, s2=FAKE)
        a.update(kw)
        return h8l(a["lg"], a["x"], a["T"], a["E"], a["k"], a["gate"], a["cap"], a["e0"],
                   a["e1"], a["d"], a["f"], a["w13"], a["s13"], a["w2"], a["s2"], a["idx"], a["w"],
                   a["counts"], a["off"], a["sp"], a["pp"], a["nk"], a["h"], a["yp"], a["y"],
                   a["ws"], a["wsb"], None)

    for key in ("w13", "s13", "w2", "s2"):
        assert call_8l(**{key: None}) == L.MOE_ERR_INVALID_ARG, key
    assert call_8l(s2=MIS) == L.MOE_ERR_MISALIGNED
    assert call_8l(d=192) == L.MOE_ERR_UNSUPPORTED
    assert call_8l(f=128) == L.MOE_ERR_UNSUPPORTED
    assert call_8l(k=9) == L.MOE_ERR_INVALID_TOPK
    assert call_8l(wsb=2047) == L.MOE_ERR_WORKSPACE
    assert call_r(k=9) == L.MOE_ERR_INVALID_TOPK
    assert call_r(gate=5) == L.MOE_ERR_INVALID_ARG
    assert call_r(y=MIS) == L.MOE_ERR_MISALIGNED
    # a workspace sized for the dispatch alone is too small once rerouting needs its scratch
    dispatch_only = ws_ok - (100 * 3 * 4 + 255) // 256 * 256 * 2 - 256
    assert call_r(wsb=dispatch_only) == L.MOE_ERR_WORKSPACE
    # the TensorList form: the same arguments with weight tables in place of the packed weights
    t = lib.moe_forward_fused_list
    assert _call_list(t, ok, w13=None) == L.MOE_ERR_INVALID_ARG
    assert _call_list(t, ok, w2=None) == L.MOE_ERR_INVALID_ARG
    assert _call_list(t, ok, w2=MIS) == L.MOE_ERR_MISALIGNED
    assert _call_list(t, ok, k=9) == L.MOE_ERR_INVALID_TOPK
    assert _call_list(t, ok, d=100) == L.MOE_ERR_UNSUPPORTED
    assert _call_list(t, ok, wsb=2047) == L.MOE_ERR_WORKSPACE


def _call_list(fn, ok, **kw):
    a = dict(ok)
    a.update(kw)
    return fn(a["lg"], a["x"], a["T"], a["E"], a["k"], a["gate"], a["cap"], a["e0"], a["e1"],
              a["d"], a["f"], a["dt"], a["w13"], a["w2"], a["idx"], a["w"], a["counts"], a["off"],
              a["sp"], a["pp"], a["nk"], a["h"], a["yp"], a["y"], a["ws"], a["wsb"], None)


def test_package_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(L, "_lib", None)
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        L.lib()


def test_header_declares_the_backward(lib):
    names = declared_functions()
    for n in ("moe_ffn_up_train", "moe_pack_weights_backward", "moe_combine_backward",
              "moe_gate_backward", "moe_ffn_down_backward", "moe_ffn_up_backward",
              "moe_wgrad_workspace_bytes", "moe_ffn_wgrad", "moe_router_backward",
              "moe_router_backward_workspace_bytes"):
        assert n in names


def test_backward_validation(lib):
    BF, F32 = L.MOE_BF16, L.MOE_F32
    # ffn_up_train: the forward's rules plus the pre-activation buffer
    up = lib.moe_ffn_up_train
    ok = [FAKE, FAKE, 4, 64, 128, 256, BF, FAKE, FAKE, FAKE, None]
    bad = list(ok); bad[9] = None
    assert up(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(ok); bad[9] = MIS
    assert up(*bad) == L.MOE_ERR_MISALIGNED
    bad = list(ok); bad[5] = 100                                  # f not a multiple of 64 (bf16)
    assert up(*bad) == L.MOE_ERR_UNSUPPORTED
    bad = list(ok); bad[3] = 1 << 24; bad[5] = 8192               # ab beyond 32-bit offsets
    assert up(*bad) == L.MOE_ERR_UNSUPPORTED
    # combine backward
    cb = lib.moe_combine_backward
    ok = [FAKE, FAKE, FAKE, FAKE, 10, 2, 64, BF, FAKE, FAKE, None]
    bad = list(ok); bad[5] = 9
    assert cb(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(ok); bad[6] = 4                                     # d * 2 bytes not a multiple of 16
    assert cb(*bad) == L.MOE_ERR_UNSUPPORTED
    bad = list(ok); bad[9] = None
    assert cb(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(ok); bad[8] = MIS
    assert cb(*bad) == L.MOE_ERR_MISALIGNED
    assert cb(None, None, None, None, 0, 2, 64, BF, None, None, None) == L.MOE_OK
    # gate backward
    gb = lib.moe_gate_backward
    ok = [FAKE, FAKE, FAKE, 10, 8, 2, 0, FAKE, None]
    bad = list(ok); bad[5] = 9
    assert gb(*bad) == L.MOE_ERR_INVALID_TOPK
    bad = list(ok); bad[6] = 5
    assert gb(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(ok); bad[7] = None
    assert gb(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(ok); bad[0] = MIS
    assert gb(*bad) == L.MOE_ERR_MISALIGNED
    # down / up backward
    db = lib.moe_ffn_down_backward
    ok = [FAKE, FAKE, 4, 64, 128, 256, BF, FAKE, FAKE, FAKE, FAKE, None]
    bad = list(ok); bad[10] = None
    assert db(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(ok); bad[8] = MIS
    assert db(*bad) == L.MOE_ERR_MISALIGNED
    bad = list(ok); bad[4] = 96
    assert db(*bad) == L.MOE_ERR_UNSUPPORTED
    ub = lib.moe_ffn_up_backward
    ok = [FAKE, FAKE, 4, 64, 128, 256, BF, FAKE, FAKE, None]
    bad = list(ok); bad[7] = None
    assert ub(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(ok); bad[2] = 0
    assert ub(*bad) == L.MOE_ERR_INVALID_ARG
    # weight gradients: workspace sized for the transposed operands (bf16)
    need = lib.moe_wgrad_workspace_bytes(1000, 8, 128, 256, BF)
    assert need >= (2 * 256 + 128) * (1000 + 8 * 31) * 2
    assert lib.moe_wgrad_workspace_bytes(1000, 8, 128, 256, F32) < 4096
    wg = lib.moe_ffn_wgrad
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, 8, 1000, 128, 256, BF, FAKE, FAKE, FAKE, need, None]
    bad = list(ok); bad[13] = need - 1
    assert wg(*bad) == L.MOE_ERR_WORKSPACE
    bad = list(ok); bad[11] = None
    assert wg(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(ok); bad[3] = None
    assert wg(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(ok); bad[2] = MIS
    assert wg(*bad) == L.MOE_ERR_MISALIGNED
    # router backward
    rb = lib.moe_router_backward
    rneed = lib.moe_router_backward_workspace_bytes(100, 64, 8)
    assert rneed >= 2 * 64 * 8 * 4
    ok = [FAKE, FAKE, FAKE, 100, 64, 8, BF, FAKE, FAKE, FAKE, rneed, None]
    bad = list(ok); bad[5] = 65
    assert rb(*bad) == L.MOE_ERR_INVALID_ARG
    bad = list(ok); bad[4] = 60
    assert rb(*bad) == L.MOE_ERR_UNSUPPORTED
    bad = list(ok); bad[10] = rneed - 1
    assert rb(*bad) == L.MOE_ERR_WORKSPACE
    bad = list(ok); bad[7] = None
    assert rb(*bad) == L.MOE_ERR_INVALID_ARG
    # pack for the backward
    pb = lib.moe_pack_weights_backward
    assert pb(FAKE, FAKE, 2, 64, 4, BF, FAKE, None) == L.MOE_ERR_UNSUPPORTED   # f * 2 bytes not a multiple of 16
    assert pb(FAKE, None, 2, 64, 64, BF, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert pb(FAKE, FAKE, 2, 64, 64, BF, MIS, None) == L.MOE_ERR_MISALIGNED
    # combine with unit weights is allowed (topk_w NULL) but still needs its other buffers
    assert lib.moe_combine(FAKE, None, None, 10, 2, 64, BF, FAKE, None) == L.MOE_ERR_INVALID_ARG


def test_ffn_plan_on_the_workload_shapes(lib):
    """The kernel choice of each FFN half, from the sizes alone (no GPU)."""
    plan = M.moe_ffn_plan
    # Mixtral-shaped prefill: few short tiles for GEMM1, 14336-deep GEMM2
    assert plan("up", 8192, 8, 4096, 14336) == "big_all"
    assert plan("down", 8192, 8, 4096, 14336) == "big_tail"
    # DeepSeek-shaped decode and the Zipf-skewed prefill (256 experts)
    assert plan("up", 1024, 256, 7168, 2048) == "stream"
    assert plan("down", 1024, 256, 7168, 2048) == "stream"
    assert plan("up", 65536, 256, 7168, 2048) == "big_ride"
    assert plan("down", 65536, 256, 7168, 2048) == "big_ride"
    # one expert-parallel rank's share: 32 local experts, capacity 320
    rows = M.moe_max_rows(16384, 2, 32, 320)
    assert rows == 10240
    assert plan("up", rows, 32, 4096, 1536) == "wide"
    assert plan("down", rows, 32, 4096, 1536) == "big_all"
    assert plan("up", 128, 8, 128, 256, dtype="f32") == "f32"
    assert plan("up", 0, 8, 128, 256) == "none"
    with pytest.raises(ValueError):
        plan("up", 10, 0, 128, 256)


def test_ffn_plan_falls_back_when_an_operand_reaches_4_gib(lib):
    """The pipelined kernels use 32-bit byte offsets for the activations, one
    expert's weights and the output: once max_rows x max(d, f) bf16 elements
    reach 4 GiB the pass takes the 64-bit-addressed streaming kernel."""
    plan = M.moe_ffn_plan
    lim = 1 << 32
    # Mixtral shape: the output h of GEMM1 (max_rows x 14336) crosses first
    r = (lim - 1) // (14336 * 2)
    assert r * 14336 * 2 < lim <= (r + 1) * 14336 * 2
    assert plan("up", r, 8, 4096, 14336) == "big_all"
    assert plan("up", r + 1, 8, 4096, 14336) == "stream (operands of 4 GiB or more)"
    assert plan("down", r + 1, 8, 4096, 14336) == "stream (operands of 4 GiB or more)"
    # DeepSeek shape: the output y_perm of GEMM2 (max_rows x 7168) crosses first
    r = (lim - 1) // (7168 * 2)
    assert plan("down", r, 256, 7168, 2048) == "big_ride"
    assert plan("down", r + 1, 256, 7168, 2048) == "stream (operands of 4 GiB or more)"
    assert plan("up", r + 1, 256, 7168, 2048) == "stream (operands of 4 GiB or more)"
    # one expert's weights of 4 GiB or more
    assert plan("up", 4096, 1, 16384, 65536) == "stream (operands of 4 GiB or more)"
