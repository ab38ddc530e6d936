"""The layer from a C program alone: tests/c_forward.c (compiled here with gcc against
include/lc_moe.h, liblc_moe.so and the HIP runtime, no Python or PyTorch in its process)
allocates its buffers with hipMalloc and runs lc_moe_forward.  Its picks equal the oracle's,
its output is within the bf16 bound of the oracle on every token, and all of its outputs
equal bitwise those of the same call made through the Python binding."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from tests.gpu_common import BF16_TOL, adhoc, audited, make_case, oracle_forward, rel_l2, say, worst_token_rel

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mixture_experts_layer_router_amd")


def build(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    exe = tmp_path / "c_forward"
    cmd = [gcc, "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-isystem", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "c_forward.c"), "-o", str(exe),
           "-L", PKG, "-llc_moe", f"-Wl,-rpath,{PKG}", "-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.parametrize("T,d,I", [(64, 512, 256), (700, 320, 192)])
def test_forward_from_c(tmp_path, T, d, I):
    """T=64: the few-row kernels; T=700: the 320-row pipelined form with ragged tiles."""
    import torch
    import mixture_experts_layer_router_amd as lm
    exe = build(tmp_path)
    wl = adhoc(name=f"cabi_{T}", T=T, d=d, N=12, Z=6, K=5, I=I, seed_key=(960, T), expert_std=1 / np.sqrt(d))
    say(f"forward from C: T={T} d={d} I={I} N={wl.N} Z={wl.Z} K={wl.K}")
    case = make_case(wl, ri=audited(wl))
    raw = lambda t: t.contiguous().view(torch.uint8).cpu().numpy().tobytes()  # noqa: E731
    for name, t in (("x", case.x), ("w_router", case.w_router), ("bias", case.bias), ("w_gate", case.w["gate"]),
                    ("w_up", case.w["up"]), ("w_down", case.w["down"])):
        (tmp_path / f"{name}.bin").write_bytes(raw(t))
    r = subprocess.run([str(exe), str(tmp_path), str(T), str(d), str(wl.N), str(wl.Z), str(wl.K), str(I)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    y_bits = np.fromfile(tmp_path / "y.bin", np.uint16).reshape(T, d)
    idx = np.fromfile(tmp_path / "idx.bin", np.int32).reshape(T, wl.K)
    gate = np.fromfile(tmp_path / "gate.bin", np.float32).reshape(T, wl.K)
    load = np.fromfile(tmp_path / "load.bin", np.int32)
    ref = oracle_forward(case)
    np.testing.assert_array_equal(idx, ref["idx"])
    y = (y_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err, worst = rel_l2(y, ref["y"]), worst_token_rel(y, ref["y"])
    say(f"   rel L2 {err:.2e} (worst token {worst:.2e})")
    assert err <= BF16_TOL and worst <= BF16_TOL
    out = lm.forward(case.x, case.w_router, case.bias, case.w["gate"], case.w["up"], case.w["down"], wl.K)
    assert np.array_equal(out["y"].view(torch.int16).cpu().numpy().view(np.uint16), y_bits)
    assert np.array_equal(out["topk_idx"].cpu().numpy(), idx)
    assert np.array_equal(out["topk_gate"].cpu().numpy().view(np.uint32), gate.view(np.uint32))
    assert np.array_equal(out["load"].cpu().numpy(), load)
