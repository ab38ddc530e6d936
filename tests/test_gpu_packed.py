"""Packed bf16 expert weights on the GPU: lc_moe_pack_weights writes the documented tile
layout (checked against an independent re-layout of the weights in numpy, bit for bit,
including the zero padding of ragged n-tiles), and the layer run on the packed weights
equals the layer run on the row-major weights bit for bit wherever both run the pipelined
kernel -- the packed form only changes where that kernel reads each weight from.  Where the
row-major weights take the whole-line few-row kernel instead, which adds the K steps in
another order, both layers are checked against the oracle and against each other."""
import numpy as np
import pytest

from inputs import configs
from tests.gpu_common import BF16_TOL, adhoc, audited, make_case, oracle_forward, rel_l2, say, to_np

pytestmark = pytest.mark.gpu


def swz4(r):
    return (((r >> 1) & 1) << 1) ^ ((r >> 2) & 1) ^ (((r >> 3) & 1) << 1)


def packed_reference(wg, wu, wd):
    """The documented layout, built from the row-major uint16 arrays: gate/up region
    [N][ceil(I/128)][d/32][256 rows][32 bf16], then (256-byte aligned) the down region
    [N][ceil(d/256)][I/32][256 rows][32 bf16]; row r's 8-column chunk c in slot c ^ swz4(r)."""
    N, I, d = wg.shape

    def tiles(mats, rows_per_mat, R, C):
        nt = -(-R // rows_per_mat)
        out = np.zeros((N, nt, C // 32, 256, 4, 8), dtype=np.uint16)
        for t in range(nt):
            for m, mat in enumerate(mats):
                r0 = t * rows_per_mat
                rows = mat[:, r0:r0 + rows_per_mat, :]                   # [N, <=rows, C]
                blk = rows.reshape(N, rows.shape[1], C // 32, 4, 8)      # [N, row, kt, chunk, 8]
                for rr in range(rows.shape[1]):
                    r = m * rows_per_mat + rr
                    for c in range(4):
                        out[:, t, :, r, c ^ swz4(r), :] = blk[:, rr, :, c, :]
        return out.reshape(-1)

    gu = tiles((wg, wu), 128, I, d)
    dn = tiles((wd,), 256, d, I)
    pad = (-(gu.size * 2)) % 256 // 2
    return np.concatenate([gu, np.zeros(pad, dtype=np.uint16), dn])


def test_pack_layout_bit_exact():
    import mixture_experts_layer_router_amd as lm
    import torch
    for (N, d, I) in [(3, 288, 160), (2, 64, 32)]:
        say(f"pack layout N={N} d={d} I={I}")
        g = torch.Generator(device="cuda").manual_seed(7)
        w = [torch.randn(s, generator=g, device="cuda").to(torch.bfloat16) for s in ((N, I, d), (N, I, d), (N, d, I))]
        packed = lm.pack_weights(*w)
        got = packed.cpu().numpy().view(np.uint16)
        ref = packed_reference(*[t.cpu().view(torch.int16).numpy().view(np.uint16) for t in w])
        assert got.size == ref.size
        assert np.array_equal(got, ref)


def run_both(case, K):
    """The layer on the row-major weights, and through the low-level call with the row-major
    pointers NULL and the packed weights set (so the FFN can only have read the packed form)."""
    import torch
    import mixture_experts_layer_router_amd as lm
    w, wl = case.w, case.wl
    a = lm.forward(case.x, case.w_router, case.bias, w["gate"], w["up"], w["down"], K)
    packed = lm.pack_weights(w["gate"], w["up"], w["down"])
    T, dev = case.x.shape[0], case.x.device
    shape = lm.make_shape(T, wl.d, wl.N, wl.Z, K, wl.I, lm.BF16)
    b = dict(y=torch.empty_like(case.x), topk_idx=torch.empty((T, K), dtype=torch.int32, device=dev),
             topk_gate=torch.empty((T, K), dtype=torch.float32, device=dev),
             load=torch.empty(wl.N + wl.Z, dtype=torch.int32, device=dev))
    lm.lc_moe_forward(shape, case.x, lm._weights(case.w_router, case.bias, None, None, None, None, packed),
                      b["y"], b["topk_idx"], b["topk_gate"], b["load"], lm.workspace_for(shape, dev))
    return a, b


def line_kernel_runs(T, d, I):
    """Whether the row-major weights take the whole-line few-row kernel in either GEMM
    (layers of at most 256 tokens; gate/up needs d % 64 == 0, down I % 64 == 0)."""
    return T <= 256 and (d % 64 == 0 or I % 64 == 0)


def assert_same(a, b):
    import torch
    for k in ("topk_idx", "topk_gate", "load"):
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(a["y"].view(torch.int16), b["y"].view(torch.int16))


def assert_pair(case, a, b, tokens=None):
    """Bit for bit where both formats run the same kernel; otherwise identical routing and
    both outputs within the bf16 tolerance of the oracle (on `tokens`, all by default)."""
    import torch
    wl = case.wl
    if not line_kernel_runs(case.x.shape[0], wl.d, wl.I):
        assert_same(a, b)
        return
    for k in ("topk_idx", "topk_gate", "load"):
        assert torch.equal(a[k], b[k]), k
    ref = oracle_forward(case, tokens=tokens)
    sel = slice(None) if tokens is None else tokens
    ya, yb = to_np(a["y"])[sel], to_np(b["y"])[sel]
    ea, eb, eab = rel_l2(ya, ref["y"]), rel_l2(yb, ref["y"]), rel_l2(ya, yb)
    say(f"  row-major vs oracle {ea:.2e}, packed vs oracle {eb:.2e}, row-major vs packed {eab:.2e}")
    assert ea <= BF16_TOL and eb <= BF16_TOL


@pytest.mark.parametrize("T,d,I,N,Z,K", [(300, 256, 160, 12, 5, 4), (96, 288, 384, 40, 20, 6),
                                         (1, 64, 32, 3, 1, 2), (1200, 128, 96, 6, 2, 3)])
def test_forward_packed_matches_row_major(T, d, I, N, Z, K):
    """Ragged gate/up n-tiles (I % 128), ragged down n-tiles (d % 256), one token, and
    experts with more than 320 rows (two M-tiles)."""
    wl = adhoc(name=f"pk{T}", T=T, d=d, N=N, Z=Z, K=K, I=I, seed_key=(411, T), expert_std=1 / np.sqrt(d))
    say(f"packed forward T={T} d={d} I={I} N={N} Z={Z} K={K}")
    case = make_case(wl, ri=audited(wl))
    a, b = run_both(case, K)
    if T == 1200:
        assert int(to_np(a["load"])[:N].max()) > 320
    assert_pair(case, a, b)


@pytest.mark.parametrize("name", ["decode_T64_z33", "prefill", "skewed"])
def test_forward_packed_full_size_matches_row_major(name):
    wl = configs.get(name)
    say(f"packed forward full size: {wl.description}")
    case = make_case(wl)
    a, b = run_both(case, wl.K)
    assert_pair(case, a, b, tokens=list(range(0, wl.T, max(1, wl.T // 6))))
