"""The C-ABI library loads without a GPU, exports every declared entry point, and rejects
bad arguments on the host with the documented status before touching the device."""
import ctypes
import os
import re

import pytest

import mixture_experts_layer_router_amd as lm

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "lc_moe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lc_moe_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 17
    lib = lm.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(lm.EXPORTED)


def test_status_and_stage_strings():
    for s in range(7):
        assert lm.status_str(s)
    assert lm.status_str(99) == "unknown status"
    assert [lm.stage_name(i) for i in range(lm.NUM_STAGES)] == ["route", "permute", "gate_up", "down", "combine"]
    assert lm.stage_name(5) == "unknown"


def good_shape():
    return lm.make_shape(T=64, d=128, N=8, Z=4, K=2, I=256, dtype=lm.BF16)


def test_workspace_size():
    s = good_shape()
    n = lm.lc_moe_workspace_size(s)
    assert n > 0 and n % 256 == 0
    # covers at least the FFN intermediates: T*K rows of I and of d bf16 values
    assert n >= 64 * 2 * (256 + 128) * 2
    bad = [dict(T=0), dict(K=13), dict(Z=-1), dict(d=100), dict(I=12), dict(dtype=7), dict(N=3000, Z=0, K=2),
           dict(N=2048, Z=2049), dict(T=1 << 28, K=8)]
    for kw in bad:
        args = dict(T=64, d=128, N=8, Z=4, K=2, I=256, dtype=lm.BF16)
        args.update(kw)
        assert lm.lc_moe_workspace_size(lm.make_shape(**args)) == 0, kw
    assert lm.lc_moe_workspace_size(lm.make_shape(T=64, d=132, N=8, Z=0, K=8, I=4, dtype=lm.F32)) > 0
    # grid limit: one workgroup of 256 work-items per pick in lc_moe_permute's row gather
    # needs T*K*256 <= 2^32 - 1
    assert lm.lc_moe_workspace_size(lm.make_shape((1 << 21) - 1, 128, 8, 4, 8, 256, lm.BF16)) > 0
    assert lm.lc_moe_workspace_size(lm.make_shape(1 << 21, 128, 8, 4, 8, 256, lm.BF16)) == 0


P = 1 << 20           # fake, 16-byte aligned device addresses: validation never dereferences
MIS = P + 4           # misaligned


def call_route(shape, x=P, wr=P, b=P, idx=P, gate=P, ws=P, nbytes=None):
    nb = lm.lc_moe_workspace_size(good_shape()) if nbytes is None else nbytes
    return lm.lib().lc_moe_route(ctypes.byref(shape) if shape is not None else None, x, wr, b, idx, gate,
                                ws, nb, None)


def test_route_validation():
    s = good_shape()
    assert call_route(None) == 1
    assert call_route(s, x=None) == 1
    assert call_route(s, gate=None) == 1
    assert call_route(s, wr=MIS) == 4
    assert call_route(s, ws=None) == 1
    assert call_route(s, nbytes=100) == 5
    assert call_route(lm.make_shape(64, 128, 8, 4, 2, 256, 5)) == 3
    assert call_route(lm.make_shape(64, 128, 8, 4, 13, 256, lm.BF16)) == 2


def test_expert_load_permute_forward_validation():
    s = good_shape()
    nb = lm.lc_moe_workspace_size(s)
    L = lm.lib()
    sp = ctypes.byref(s)
    assert L.lc_moe_expert_load(sp, None, P, None, P, nb, None) == 1
    assert L.lc_moe_expert_load(sp, P, P, MIS, P, nb, None) == 4
    assert L.lc_moe_expert_load(sp, P, P, None, P, nb - 1, None) == 5
    assert L.lc_moe_permute(sp, P, P, None, P, P, None, None, P, nb, None) == 1
    assert L.lc_moe_permute(sp, None, P, P, P, P, P, None, P, nb, None) == 1   # x needed for x_perm
    assert L.lc_moe_permute(sp, P, P, P, P, MIS, None, None, P, nb, None) == 4
    w = lm.Weights(P, P, P, P, P)
    assert L.lc_moe_forward(sp, P, None, P, None, None, None, P, nb, None) == 1
    assert L.lc_moe_forward(sp, P, ctypes.byref(w), None, None, None, None, P, nb, None) == 1
    w2 = lm.Weights(P, P, MIS, P, P)
    assert L.lc_moe_forward(sp, P, ctypes.byref(w2), P, None, None, None, P, nb, None) == 4
    assert L.lc_moe_forward(sp, P, ctypes.byref(w), P, None, None, None, P, nb - 256, None) == 5
    bad = lm.make_shape(64, 128, 8, 4, 2, 256, lm.F32)
    bad.I = 6
    assert L.lc_moe_forward(ctypes.byref(bad), P, ctypes.byref(w), P, None, None, None, P, nb, None) == 2
    ev = (ctypes.c_void_p * 6)(*([P] * 5 + [0]))
    assert L.lc_moe_forward_staged(sp, P, ctypes.byref(w), P, None, None, None, P, nb, None,
                                   ctypes.cast(ev, ctypes.c_void_p)) == 1


def test_bias_update_validation():
    s = good_shape()
    g = lm.Pid(0.5, 0.05, 0.0)
    f = lm.lib().lc_moe_bias_update
    assert f(None, ctypes.byref(g), P, P, P, P, P, None) == 1
    assert f(ctypes.byref(s), None, P, P, P, P, P, None) == 1
    assert f(ctypes.byref(s), ctypes.byref(g), None, P, P, P, P, None) == 1
    assert f(ctypes.byref(s), ctypes.byref(g), P, P, P, P, None, None) == 1
    assert f(ctypes.byref(s), ctypes.byref(g), P, MIS, P, P, P, None) == 4
    assert f(ctypes.byref(lm.make_shape(64, 128, 8, 4, 13, 256, lm.BF16)), ctypes.byref(g), P, P, P, P, P,
             None) == 2


def test_fp8_size_and_quantize_validation():
    s = lm.make_shape(T=64, d=128, N=8, Z=4, K=2, I=256, dtype=lm.BF16)
    n = lm.lc_moe_fp8_weights_size(s)
    # codes (one byte per weight, gate/up n-tiles of 128 rows, down n-tiles of 256) + scales
    assert n >= 8 * (2 * 256 * 128 + 256 * 256) and n % 256 == 0
    assert lm.lc_moe_fp8_weights_size(lm.make_shape(64, 128, 8, 4, 2, 256, lm.F32)) == 0
    assert lm.lc_moe_fp8_weights_size(lm.make_shape(64, 136, 8, 4, 2, 256, lm.BF16)) == 0  # d % 32
    f = lm.lib().lc_moe_quantize_weights
    assert f(ctypes.byref(lm.make_shape(64, 128, 8, 4, 2, 256, lm.F32)), P, P, P, P, n, None) == 3
    assert f(ctypes.byref(lm.make_shape(64, 136, 8, 4, 2, 256, lm.BF16)), P, P, P, P, n, None) == 2
    assert f(ctypes.byref(s), None, P, P, P, n, None) == 1
    assert f(ctypes.byref(s), P, P, MIS, P, n, None) == 4
    assert f(ctypes.byref(s), P, P, P, P, n - 1, None) == 5


def test_packed_size_and_pack_validation():
    s = lm.make_shape(T=64, d=128, N=8, Z=4, K=2, I=256, dtype=lm.BF16)
    n = lm.lc_moe_packed_weights_size(s)
    # gate/up: 2 n-tiles x 4 K steps x 16 KB; down: 1 n-tile x 8 K steps x 16 KB, per expert
    assert n == 8 * (2 * 4 + 1 * 8) * 16384
    assert lm.lc_moe_packed_weights_size(lm.make_shape(64, 128, 8, 4, 2, 256, lm.F32)) == 0
    assert lm.lc_moe_packed_weights_size(lm.make_shape(64, 136, 8, 4, 2, 256, lm.BF16)) == 0  # d % 32
    # ragged n-tiles are zero-padded to whole blocks: I=160 -> 2 gate/up n-tiles of 9 K steps,
    # d=288 -> 2 down n-tiles of 5 K steps, 3 experts
    assert lm.lc_moe_packed_weights_size(lm.make_shape(1, 288, 3, 0, 1, 160, lm.BF16)) == \
        3 * (2 * 9 + 2 * 5) * 16384
    f = lm.lib().lc_moe_pack_weights
    assert f(ctypes.byref(lm.make_shape(64, 128, 8, 4, 2, 256, lm.F32)), P, P, P, P, n, None) == 3
    assert f(ctypes.byref(lm.make_shape(64, 136, 8, 4, 2, 256, lm.BF16)), P, P, P, P, n, None) == 2
    assert f(ctypes.byref(s), None, P, P, P, n, None) == 1
    assert f(ctypes.byref(s), P, P, MIS, P, n, None) == 4
    assert f(ctypes.byref(s), P, P, P, P, n - 1, None) == 5


def test_forward_weight_format_validation():
    """fp8 and packed weights are exclusive, and each needs a bf16 shape that has that form;
    all of it is decided on the host before anything is enqueued."""
    L = lm.lib()
    sp = ctypes.byref(good_shape())
    nb = lm.lc_moe_workspace_size(good_shape())
    both = lm.Weights(P, P, None, None, None, P, P)
    assert L.lc_moe_forward(sp, P, ctypes.byref(both), P, None, None, None, P, nb, None) == 3
    packed = lm.Weights(P, P, None, None, None, None, P)
    f32 = lm.make_shape(64, 128, 8, 4, 2, 256, lm.F32)
    assert L.lc_moe_forward(ctypes.byref(f32), P, ctypes.byref(packed), P, None, None, None, P,
                            lm.lc_moe_workspace_size(f32), None) == 3
    odd = lm.make_shape(64, 136, 8, 4, 2, 256, lm.BF16)
    assert L.lc_moe_forward(ctypes.byref(odd), P, ctypes.byref(packed), P, None, None, None, P,
                            lm.lc_moe_workspace_size(odd), None) == 2
    mis = lm.Weights(P, P, None, None, None, None, MIS)
    assert L.lc_moe_forward(sp, P, ctypes.byref(mis), P, None, None, None, P, nb, None) == 4
    # FP8 activations need the FP8 weights, and d, I multiples of 64
    act_only = lm.Weights(P, P, P, P, P, None, None, 1)
    assert L.lc_moe_forward(sp, P, ctypes.byref(act_only), P, None, None, None, P, nb, None) == 3
    act = lm.Weights(P, P, None, None, None, P, None, 1)
    d96 = lm.make_shape(64, 96, 8, 4, 2, 256, lm.BF16)     # d % 32 == 0 (FP8 weights) but d % 64 != 0
    assert lm.lc_moe_fp8_weights_size(d96) > 0
    assert L.lc_moe_forward(ctypes.byref(d96), P, ctypes.byref(act), P, None, None, None, P,
                            lm.lc_moe_workspace_size(d96), None) == 2
    # the FP8 MFMA layer addresses its activation matrices with 32-bit offsets: T*K*I < 2^31
    big = lm.make_shape(1 << 20, 64, 8, 4, 8, 512, lm.BF16)   # T*K*I = 2^32, T*K = 2^23
    assert lm.lc_moe_workspace_size(big) > 0 and lm.lc_moe_fp8_weights_size(big) > 0
    assert L.lc_moe_forward(ctypes.byref(big), P, ctypes.byref(act), P, None, None, None, P,
                            lm.lc_moe_workspace_size(big), None) == 2
    ok = lm.make_shape(1 << 16, 64, 8, 4, 8, 512, lm.BF16)    # T*K*I = 2^28
    nb_ok = lm.lc_moe_workspace_size(ok)
    assert L.lc_moe_forward(ctypes.byref(ok), P, ctypes.byref(act), P, None, None, None, P, nb_ok - 1, None) == 5


def test_quantize_activations_validation():
    f = lm.lib().lc_moe_quantize_activations
    assert f(P, 4, 96, P, P, None) == 2          # cols % 64
    assert f(P, 4, 0, P, P, None) == 2
    assert f(P, 4, 16384 + 64, P, P, None) == 2
    assert f(P, -1, 128, P, P, None) == 2
    assert f(P, 1 << 24, 128, P, P, None) == 2
    assert f(None, 4, 128, P, P, None) == 1
    assert f(P, 4, 128, P, None, None) == 1
    assert f(P, 4, 128, MIS, P, None) == 4
    assert f(None, 0, 128, None, None, None) == 0  # nothing to do



HIP_MAPS = r"""
import sys
sys.path.insert(0, {root!r})
{first}
paths = set()
for line in open('/proc/self/maps'):
    f = line.split()
    if len(f) >= 6 and 'libamdhip64' in f[-1]:
        paths.add(f[-1])
print(len(paths))
"""


def _hip_runtimes(first):
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = HIP_MAPS.format(root=root, first=first)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, cwd="/tmp")
    assert r.returncode == 0, r.stderr[-2000:]
    return int(r.stdout.strip().splitlines()[-1])


def test_binding_loads_one_hip_runtime():
    """torch's wheel carries its own HIP runtime under the same soname as the system one
    liblc_moe.so links to; a process that maps both crashed in a GPU run.  The binding
    imports torch before opening the library, so the library binds to the runtime already
    loaded and the process maps exactly one.  The other order (library first) maps two,
    which shows the check can fail."""
    assert _hip_runtimes("import mixture_experts_layer_router_amd as lm; lm.lib()") == 1
    lib = os.path.join(os.path.dirname(os.path.abspath(lm.__file__)), "liblc_moe.so")
    wrong = f"import ctypes; ctypes.CDLL({lib!r}); import torch"
    assert _hip_runtimes(wrong) == 2


def test_forward_noalloc_validation():
    """The allocation-free forward rejects bad shapes and shapes whose workspace exceeds its
    static array on the host, before it looks up the array or enqueues anything."""
    L = lm.lib()
    w = lm.Weights(P, P, P, P, P)
    bad = lm.make_shape(64, 128, 8, 4, 13, 256, lm.BF16)
    assert L.lc_moe_forward_noalloc(ctypes.byref(bad), P, ctypes.byref(w), P, None, None, None, None) == 2
    prefill = lm.make_shape(16384, 6144, 512, 256, 12, 2048, lm.BF16)
    assert lm.lc_moe_workspace_size(prefill) > lm.STATIC_WORKSPACE_BYTES
    assert L.lc_moe_forward_noalloc(ctypes.byref(prefill), P, ctypes.byref(w), P, None, None, None, None) == 5
    for T in (64, 128, 256):   # every decode batch of the prefill layer fits
        assert lm.lc_moe_workspace_size(lm.make_shape(T, 6144, 512, 256, 12, 2048, lm.BF16)) <= \
            lm.STATIC_WORKSPACE_BYTES


def test_backward_validation():
    """lc_moe_ffn_backward: bf16 layers with d and I multiples of 32, every pointer needed,
    a large enough workspace; decided on the host before anything is enqueued."""
    L = lm.lib()
    s = good_shape()
    nb = lm.lc_moe_backward_workspace_size(s)
    assert nb > 0 and nb % 256 == 0
    assert lm.lc_moe_backward_workspace_size(lm.make_shape(64, 128, 8, 4, 2, 256, lm.F32)) == 0
    assert lm.lc_moe_backward_workspace_size(lm.make_shape(64, 136, 8, 4, 2, 256, lm.BF16)) == 0
    w = lm.Weights(P, P, P, P, P)
    sp = ctypes.byref(s)
    args = lambda **kw: [kw.get(k, P) for k in ("x", "idx", "gate", "dy", "dx", "dwg", "dwu", "dwd")]  # noqa: E731

    def call(shape=sp, weights=ctypes.byref(w), ws=P, nbytes=nb, **kw):
        x, idx, gate, dy, dx, dwg, dwu, dwd = args(**kw)
        return L.lc_moe_ffn_backward(shape, x, weights, idx, gate, dy, dx, dwg, dwu, dwd, ws, nbytes, None)

    assert call(shape=ctypes.byref(lm.make_shape(64, 128, 8, 4, 2, 256, lm.F32))) == 3
    assert call(shape=ctypes.byref(lm.make_shape(64, 136, 8, 4, 2, 256, lm.BF16))) == 2
    assert call(weights=None) == 1
    assert call(dy=None) == 1
    assert call(dwd=None) == 1
    assert call(dx=MIS) == 4
    assert call(ws=None) == 1
    assert call(nbytes=nb - 1) == 5
    assert call(weights=ctypes.byref(lm.Weights(P, P, None, P, P))) == 1
