"""hinm_spmm on the GPU against the float64 oracle product.

Bar: |Y - Y_o| <= 1e-2 (|W_hat| |X|) elementwise and relative Frobenius error
<= 5e-3, Y_o = (W (.) M) X in float64 from the oracle's own mask.  Every
output element is compared, at every batch (the float64 product of the
largest case takes about a second on the host).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle.hinm as oh
import synth
from helpers import bits_of, check_y, oracle_pack

pytestmark = pytest.mark.gpu
hinm = pytest.importorskip("structured_sparse_gemm_amd")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DEV = torch.device("cuda:0")


class Case:
    """A workload packed on both sides; products checked at several batches."""

    def __init__(self, w: synth.Workload, v_s=None):
        self.w = w
        self.v_s = w.v_s if v_s is None else v_s
        print(f"[spmm] {w.name} {w.cout}x{w.cin} R={w.tile_rows} t_s={w.t_s} v_s={self.v_s}", flush=True)
        self.pk = hinm.pack(w.w_bf16.to(DEV), w.importance.to(DEV), w.tile_rows, w.t_s, self.v_s, w.perm.to(DEV))
        self.p, _, inter = oracle_pack(w, v_s)
        self.w_hat = oh.masked_weight(bits_of(w.w_bf16), inter["mask"])

    def check(self, batch: int, seed: int = 0, rows=None, x=None, label=""):
        if x is None:
            g = torch.Generator().manual_seed(1000 + seed)
            x = torch.randn(self.w.cin, batch, generator=g).to(torch.bfloat16)
        print(f"[spmm]   batch={batch} rows={'all' if rows is None else len(rows)} {label}", flush=True)
        y = hinm.spmm(self.pk, x.to(DEV))
        torch.cuda.synchronize()
        xf = synth.as_f64(x)
        wh = self.w_hat if rows is None else self.w_hat[rows]
        ref = oh.spmm(wh, xf)
        scale = np.abs(wh) @ np.abs(xf)
        got = y if rows is None else y[torch.as_tensor(rows, device=DEV)]
        return check_y(got, ref, scale, f"{self.w.name} batch {batch}")


def test_spmm_tiny():
    w = synth.tiny()
    c = Case(w)
    c.check(8, x=w.x_bf16)
    # Secondary oracle on the unrounded fp32 weight and activations: the bf16
    # rounding of the inputs stays inside the same bound.
    y = hinm.spmm(c.pk, w.x_bf16.to(DEV))
    torch.cuda.synchronize()
    _, _, inter = oracle_pack(w)
    wf = np.where(inter["mask"], w.w_f32.numpy().astype(np.float64), 0.0)
    xf = w.x_f32.numpy().astype(np.float64)
    check_y(y, wf @ xf, np.abs(wf) @ np.abs(xf), "tiny vs fp32 inputs")


def test_spmm_q_proj_decode():
    w = synth.q_proj(batch=16)
    Case(w).check(16, x=w.x_bf16)


def test_spmm_up_proj_prefill():
    w = synth.up_proj(batch=2048)
    Case(w).check(2048, x=w.x_bf16)


@pytest.mark.parametrize("batch", [16, 2048])
def test_spmm_down_proj(batch):
    w = synth.down_proj(batch=batch)
    Case(w).check(batch, x=w.x_bf16)


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_spmm_down_proj_sweep(idx):
    g = json.load(open(os.path.join(GOLDEN, "down_proj_boundary.json")))["results"][idx]
    c = Case(synth.down_proj_sweep(g["t_s"], batch=1), v_s=g["v_s"])
    for b in (1, 64, 512):
        c.check(b, seed=b)


@pytest.mark.parametrize("layer,proj", [(0, 0), (13, 4), (31, 6)])
def test_spmm_stack_layers(layer, proj):
    """The 7B-shaped stack's shapes at every batch of its sweep that changes the launch shape, plus
    3000 (a prefill batch past 2048 that is not a multiple of the 256-token block)."""
    c = Case(synth.stack_layer(layer, proj, batch=1))
    for b in (1, 16, 64, 256, 1024, 2048, 3000, 4096):
        c.check(b, seed=b)


def test_spmm_ragged_batches():
    c = Case(synth.small(192, 264, 64, 0.6, 0.35, 1, seed=4))
    for b in (1, 2, 3, 8, 15, 17, 31, 33, 63, 64, 65, 100, 1000):
        c.check(b, seed=b)


@pytest.mark.parametrize("args", [
    (64, 100, 16, 0.5, 0.25), (96, 132, 48, 0.6, 0.3), (128, 256, 64, 0.0, 0.0),
    (128, 256, 64, 0.75, 0.75), (128, 256, 64, 0.75, 0.5), (160, 4, 32, 0.5, 0.0), (64, 300, 64, 0.9, 0.85),
])
def test_spmm_edge_shapes(args):
    cout, cin, R, t, v = args
    c = Case(synth.small(cout, cin, R, t, v, 1, seed=cout + cin))
    for b in (1, 16, 24, 40, 70):
        c.check(b, seed=b)


def test_spmm_strided_and_unaligned_x():
    c = Case(synth.small(128, 320, 64, 0.6, 0.3, 1, seed=12))
    g = torch.Generator().manual_seed(3)
    big = torch.randn(320, 40, generator=g).to(torch.bfloat16)
    c.check(24, x=big[:, :24], label="ldx=40")                       # ldx > batch, 16-byte rows
    raw = torch.randn(320 * 24 + 1, generator=g).to(torch.bfloat16)
    xv = raw[1:].view(320, 24)                                       # 2-byte aligned only
    xd =  torch.empty(320 * 24 + 1, dtype=torch.bfloat16, device=DEV)
    xd[1:].copy_(xv.reshape(-1).to(DEV))
    xdv = xd[1:].view(320, 24)
    assert xdv.data_ptr() % 16 != 0
    y = hinm.spmm(c.pk, xdv)
    torch.cuda.synchronize()
    xf = synth.as_f64(xv)
    check_y(y, c.w_hat @ xf, np.abs(c.w_hat) @ np.abs(xf), "unaligned x")
    out = torch.full((128, 40), 7.0, dtype=torch.bfloat16, device=DEV)
    hinm.spmm(c.pk, xdv, out=out[:, :24])
    torch.cuda.synchronize()
    check_y(out[:, :24], c.w_hat @ xf, np.abs(c.w_hat) @ np.abs(xf), "ldy=40")
    assert (out[:, 24:] == 7.0).all(), "columns past the batch were written"


def test_spmm_deterministic():
    c = Case(synth.small(512, 1024, 64, 0.7, 0.45, 1, seed=8))
    for b in (4, 16, 300):
        x = torch.randn(1024, b, generator=torch.Generator().manual_seed(b)).to(torch.bfloat16).to(DEV)
        y1 = hinm.spmm(c.pk, x).clone()
        y2 = hinm.spmm(c.pk, x)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_spmm_permutation_invariance():
    """Relabelling input channels of W, importance, perm and X gives a bitwise-identical Y."""
    w = synth.small(256, 512, 64, 0.6, 0.3, 1, seed=21)
    x = torch.randn(512, 48, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16)
    pk = hinm.pack(w.w_bf16.to(DEV), w.importance.to(DEV), 64, 0.6, 0.3, w.perm.to(DEV))
    y = hinm.spmm(pk, x.to(DEV))
    sig = torch.from_numpy(np.random.default_rng(1).permutation(512))
    inv = torch.argsort(sig)
    perm2 = inv[w.perm.long()].to(torch.int32)
    pk2 = hinm.pack(w.w_bf16[:, sig].contiguous().to(DEV), w.importance[:, sig].contiguous().to(DEV), 64, 0.6, 0.3,
                    perm2.to(DEV))
    y2 = hinm.spmm(pk2, x[sig].contiguous().to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_spmm_empty_batch():
    c = Case(synth.small(64, 128, 64, 0.5, 0.25, 1, seed=1))
    y = hinm.spmm(c.pk, torch.empty(128, 0, dtype=torch.bfloat16, device=DEV))
    assert y.shape == (64, 0)


def test_spmm_shared_workspace_across_shapes():
    """One workspace serves products of different shapes and split counts in turn."""
    ws = torch.zeros(1 << 24, dtype=torch.uint8, device=DEV)
    cases = [Case(synth.small(256, 4096, 64, 0.75, 0.55, 1, seed=31)),
             Case(synth.small(128, 1024, 64, 0.5, 0.25, 1, seed=32)),
             Case(synth.small(96, 1024, 48, 0.5, 0.25, 1, seed=33)),      # generic path (tile_rows 48)
             Case(synth.small(4096, 1024, 64, 0.6, 0.3, 1, seed=34))]     # many tiles
    for rep in range(3):
        for c in cases:
            for b in (1, 16, 40, 100):
                x = torch.randn(c.w.cin, b, generator=torch.Generator().manual_seed(rep * 100 + b)).to(torch.bfloat16)
                y = hinm.spmm(c.pk, x.to(DEV), workspace=ws)
                torch.cuda.synchronize()
                xf = synth.as_f64(x)
                check_y(y, c.w_hat @ xf, np.abs(c.w_hat) @ np.abs(xf), f"shared ws rep {rep} batch {b}")


def test_spmm_graph_replay():
    """Products captured in a HIP graph (as the benchmark times the batch-16 point) give the eager
    results on every replay, with eager work and synchronisation between replays."""
    cases = [(Case(synth.small(256, 4096, 64, 0.75, 0.55, 1, seed=41)), 16),    # split-K decode, workspace
             (Case(synth.small(256, 4096, 64, 0.75, 0.55, 1, seed=41)), 300),   # prefill
             (Case(synth.small(96, 1024, 48, 0.5, 0.25, 1, seed=42)), 40)]      # generic split + reduce
    g_in = torch.Generator().manual_seed(7)
    xs = [torch.randn(c.w.cin, b, generator=g_in).to(torch.bfloat16).to(DEV) for c, b in cases]
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    eager = [hinm.spmm(c.pk, x, workspace=ws) for (c, _), x in zip(cases, xs)]
    torch.cuda.synchronize()
    outs = [torch.empty_like(e) for e in eager]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for (c, _), x, o in zip(cases, xs, outs):
            hinm.spmm(c.pk, x, out=o, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for (c, _), x, o in zip(cases, xs, outs):
            hinm.spmm(c.pk, x, out=o, workspace=ws)
    for rep in range(4):
        for o in outs:
            o.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16)), f"replay {rep} product {i}"
        # eager work on the same workspace between replays
        (c, _), x = cases[0], xs[0]
        assert torch.equal(hinm.spmm(c.pk, x, workspace=ws).view(torch.int16), eager[0].view(torch.int16))
        torch.cuda.synchronize()


@pytest.mark.parametrize("unaligned", [False, True])
def test_spmm_last_x_row_odd_batches(unaligned):
    """The last input channel kept in every tile (its importance raised), at
    odd and ragged batches: the gather's 16-byte loads of that row end past
    the X buffer, so its tokens must come back whole.  Unaligned: X starts 2
    bytes past a 16-byte boundary."""
    w = synth.small(128, 264, 64, 0.6, 0.35, 1, seed=21)
    w.importance[:, -1] = w.importance.max() * 4.0
    c = Case(w)
    assert (c.w_hat[:, -1] != 0).all()                                 # kept (dense) in every tile
    for b in (1, 3, 5, 7, 9, 13, 17, 23, 33, 47, 63):
        g = torch.Generator().manual_seed(b)
        x = torch.randn(264, b, generator=g).to(torch.bfloat16)
        x[-1] = torch.linspace(1.0, 2.0, b).to(torch.bfloat16)         # never zero: a lost token shows
        if unaligned:
            buf = torch.empty(264 * b + 1, dtype=torch.bfloat16, device=DEV)
            buf[1:].copy_(x.reshape(-1).to(DEV))
            xd = buf[1:].view(264, b)
        else:
            xd = x.to(DEV)
        print(f"[spmm]   last row, batch={b} unaligned={unaligned}", flush=True)
        y = hinm.spmm(c.pk, xd)
        torch.cuda.synchronize()
        xf = synth.as_f64(x)
        check_y(y, c.w_hat @ xf, np.abs(c.w_hat) @ np.abs(xf), f"last row batch {b}")


@pytest.mark.parametrize("unaligned", [False, True])
def test_spmm_decode_ragged_full_width(unaligned):
    """Split-K decode at q_proj's full 4096x4096 shape (4 K splits): ragged batches in every token-block size,
    X contiguous (rows 16-byte aligned only at multiples of 8 tokens) or starting 2 bytes past a 16-byte
    boundary; every output row checked."""
    c = Case(synth.q_proj(batch=16))
    for b in (1, 7, 8, 13, 24, 33, 47, 64):
        g = torch.Generator().manual_seed(300 + b)
        x = torch.randn(c.w.cin, b, generator=g).to(torch.bfloat16)
        if unaligned:
            buf = torch.empty(c.w.cin * b + 1, dtype=torch.bfloat16, device=DEV)
            buf[1:].copy_(x.reshape(-1).to(DEV))
            xd = buf[1:].view(c.w.cin, b)
        else:
            xd = x.to(DEV)
        print(f"[spmm]   full-width decode batch={b} unaligned={unaligned}", flush=True)
        y = hinm.spmm(c.pk, xd)
        torch.cuda.synchronize()
        xf = synth.as_f64(x)
        check_y(y, oh.spmm(c.w_hat, xf), np.abs(c.w_hat) @ np.abs(xf), f"q_proj batch {b}")


def test_spmm_decode_small_batch_x_layouts_bit_identical():
    """Batches of 1 to 63 tokens (every token-block width), X rows at every 2-byte alignment: a contiguous X
    (odd row pitch at odd batches), odd and even row strides, and X starting 2 bytes past a dword.  At batch
    1 every element is a 2-byte load; otherwise rows that are not 16-byte aligned take 16-byte loads from
    2-byte-aligned addresses (the last row's partial chunk one token early).  The product must be
    bit-identical to the same product from a copy of X with 64-token rows (the same kernel, adding the same
    terms in the same order), and within the bar of the oracle.  The last input channel is kept in every
    tile, so the end of the X buffer is exercised too."""
    w = synth.small(256, 1032, 64, 0.6, 0.35, 1, seed=31)
    w.importance[:, -1] = w.importance.max() * 4.0
    c = Case(w)
    cin = w.cin
    for b in (1, 2, 3, 4, 5, 7, 9, 15, 17, 31, 33, 45, 63):
        g = torch.Generator().manual_seed(500 + b)
        x = torch.randn(cin, b, generator=g).to(torch.bfloat16)
        ref64 = torch.zeros(cin, 64, dtype=torch.bfloat16, device=DEV)
        ref64[:, :b] = x.to(DEV)
        y_ref = hinm.spmm(c.pk, ref64[:, :b])
        xf = synth.as_f64(x)
        for ldx in sorted({b, b + 1, b + 2, 2 * b + 1}):
            for shift in (0, 1):
                buf = torch.zeros(cin * ldx + shift + 8, dtype=torch.bfloat16, device=DEV)
                xd = buf[shift:shift + cin * ldx].view(cin, ldx)[:, :b]
                xd.copy_(x.to(DEV))
                print(f"[spmm]   batch={b} ldx={ldx} base+{2 * shift} bytes", flush=True)
                y = hinm.spmm(c.pk, xd)
                torch.cuda.synchronize()
                assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), (b, ldx, shift)
        check_y(y_ref, oh.spmm(c.w_hat, xf), np.abs(c.w_hat) @ np.abs(xf), f"small batch {b}")


def test_spmm_batch1_wide_inputs():
    """Batch 1 gathers each element with a 2-byte load.  Input widths from 4100 to 16384 channels, the last
    channel kept in every tile (its element ends the X buffer): a contiguous X (rows 2 bytes apart) must
    give the same bits as the same X with 8-token rows, and both meet the oracle's bar."""
    for cin, cout in ((15872, 64), (15860, 64), (15876, 64), (16384, 64), (4100, 256)):
        w = synth.small(cout, cin, 64, 0.6, 0.35, 1, seed=cin)
        w.importance[:, -1] = w.importance.max() * 4.0
        c = Case(w)
        x = torch.randn(cin, 1, generator=torch.Generator().manual_seed(cin)).to(torch.bfloat16)
        x[-1] = 1.5                                                    # never zero: a lost element shows
        wide = torch.zeros(cin, 8, dtype=torch.bfloat16, device=DEV)
        wide[:, :1] = x.to(DEV)
        print(f"[spmm]   batch 1, cin={cin}, contiguous X and 8-token rows", flush=True)
        y = hinm.spmm(c.pk, x.to(DEV))
        y_ref = hinm.spmm(c.pk, wide[:, :1])
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), cin
        xf = synth.as_f64(x)
        check_y(y, oh.spmm(c.w_hat, xf), np.abs(c.w_hat) @ np.abs(xf), f"batch 1 cin {cin}")


@pytest.mark.parametrize("batch", [16, 100])
def test_spmm_x_beyond_32bit_offsets(batch):
    """X whose row stride puts its last row past 2^31 bytes (4096 rows of 300000 elements, 2.46 GB).
    The split decode and the batch > 64 kernel address X with 32-bit buffer offsets, so such a call
    takes the 64-bit-addressed kernels (batch <= 64: the unsplit decode; batch > 64: the generic
    LDS-gather kernel).  Every row against the oracle; the same X copied contiguous (32-bit
    kernels) meets the same bar."""
    c = Case(synth.q_proj(batch=16))
    g = torch.Generator().manual_seed(31 + batch)
    x = torch.randn(4096, batch, generator=g).to(torch.bfloat16)
    ldx = 300000
    assert (4095 * ldx + batch) * 2 > 2**31
    big = torch.zeros(4096, ldx, dtype=torch.bfloat16, device=DEV)
    big[:, :batch].copy_(x.to(DEV))
    print(f"[spmm]   batch={batch} ldx={ldx} (X past 2^31 bytes)", flush=True)
    y = hinm.spmm(c.pk, big[:, :batch])
    torch.cuda.synchronize()
    del big
    xf = synth.as_f64(x)
    ref, scale = oh.spmm(c.w_hat, xf), np.abs(c.w_hat) @ np.abs(xf)
    check_y(y, ref, scale, f"q_proj batch {batch}, X past 2^31 bytes")
    y32 = hinm.spmm(c.pk, x.to(DEV))
    torch.cuda.synchronize()
    check_y(y32, ref, scale, f"q_proj batch {batch}, contiguous X")
