"""Safety nets on the GPU: guard bands and repeatability for every entry point.

Every output buffer (and every caller workspace) is the middle of a larger
allocation whose 4 KiB guard bands on both sides hold a sentinel byte; after
each call the guards must be untouched. The shapes are ragged against the
kernels' tiles (rows, columns, K steps, partial pieces, split K), so a store
or a workspace write one element past its end shows up here. Each call is
made three times into the same buffers and must give the same bits each
time (no float atomics anywhere; integer sums are order-free)."""
import math

import numpy as np
import pytest

import oracle
import ternary_weight_linear_quant_amd as bl
from ternary_weight_linear_quant_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

DEV = torch.device("cuda:0")
GUARD = 4096
SENTINEL = 0xA5


class Guarded:
    """A tensor of `shape` and `dtype` inside a sentinel-filled allocation."""

    def __init__(self, shape, dtype):
        shape = tuple(shape) if isinstance(shape, (tuple, list)) else (shape,)
        nbytes = math.prod(shape) * torch.empty((), dtype=dtype).element_size()
        self.n = nbytes
        self.buf = torch.full((GUARD + nbytes + GUARD,), SENTINEL, dtype=torch.uint8,
                              device=DEV)
        self.t = self.buf[GUARD:GUARD + nbytes].view(dtype).view(shape)

    def intact(self):
        torch.cuda.synchronize()
        return bool((self.buf[:GUARD] == SENTINEL).all().item() and
                    (self.buf[GUARD + self.n:] == SENTINEL).all().item())

    def bits(self):
        return self.buf[GUARD:GUARD + self.n].clone()


def _three_times(call, outs):
    """Run `call` three times into the same guarded outputs: every guard
    intact after each, the same bytes each time."""
    first = None
    for _ in range(3):
        call()
        torch.cuda.synchronize()
        for i, g in enumerate(outs):
            assert g.intact(), f"guard band of output {i} overwritten"
        cur = [g.bits() for g in outs]
        if first is None:
            first = cur
        else:
            for a, b in zip(first, cur):
                assert torch.equal(a, b), "outputs differ between identical calls"
    return first


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).to(DEV) \
        .view(torch.bfloat16)


def dev_packed(p):
    return torch.from_numpy(np.ascontiguousarray(p, np.uint32).view(np.int32)).to(DEV)


def _codes(rng, N, K):
    return rng.integers(-1, 2, size=(N, K)).astype(np.int8)


# ------------------------------------------------------------ weights ----

@pytest.mark.parametrize("N,K", [(7, 64), (33, 320), (200, 4160)])
def test_weight_preparation_guards_and_repeats(N, K):
    W = dev_f32(wl.weights(60, 0, N, K))
    ws = Guarded(max(8, bl.lib().bl_quantize_weights_workspace_bytes(N, K)) // 8, torch.float64)
    pk = Guarded((N, K // 16), torch.int32)
    g = Guarded(1, torch.float32)
    _three_times(lambda: bl.quantize_weights(W, workspace=ws.t, out=(pk.t, g.t)), [pk, g, ws])
    nb = bl.lib().bl_packed_bytes_binary(N, K)
    bits = Guarded((N, nb // (4 * N)), torch.int32)
    gb = Guarded(1, torch.float32)
    _three_times(lambda: bl.quantize_weights_binary(W, workspace=ws.t, out=(bits.t, gb.t)),
                 [bits, gb, ws])
    n3 = bl.lib().bl_packed_bytes_base3(N, K)
    b3 = Guarded((N, n3 // N), torch.uint8)
    _three_times(lambda: bl.pack_base3(pk.t, K, out=b3.t), [b3])
    nt = bl.lib().bl_ste_t_bytes(N, K)
    qT = Guarded((K, nt // K), torch.uint8)
    _three_times(lambda: bl.pack_ste_t(pk.t, K, out=qT.t), [qT])


# --------------------------------------------------------- activations ----

@pytest.mark.parametrize("M,K", [(1, 64), (3, 320), (5, 8640), (300, 2560), (2, 28672)])
@pytest.mark.parametrize("fused", [False, True])
def test_act_quant_guards_and_repeats(M, K, fused):
    x = dev_bf16(wl.activations(61, 0, M, K))
    gain = dev_bf16(wl.rms_gain(61, 0, K)) if fused else None
    xq = Guarded((M, K), torch.int8)
    xs = Guarded(M, torch.float32)
    _three_times(lambda: bl.quantize_acts(x, gain, out=(xq.t, xs.t)), [xq, xs])


# ------------------------------------------------------------ products ----

# One-token (cached, streamed, partial pieces), GEMV (ragged rows), wide GEMV,
# GEMM large tiles (ragged M, N, half K step), K groups, split K.
PRODUCT_CASES = [
    (1, 320, 200, 4), (1, 4160, 7, 4), (1, 12288, 33, 4), (1, 8256, 31, 4),
    (3, 2560, 257, 1), (16, 6912, 100, 1), (9, 1024, 6150, 1),
    (37, 3200, 300, 3), (64, 8192, 129, 3),
    (2000, 320, 4000, 2), (1935, 448, 5000, 2), (4050, 704, 1920, 2),
    (100, 2560, 300, 2), (70, 28672, 65, 2), (33, 8192, 1000, 2), (500, 3136, 8640, 2),
]


@pytest.mark.parametrize("M,K,N,path", PRODUCT_CASES)
def test_bitlinear_guards_and_repeats(M, K, N, path):
    rng = np.random.default_rng(M + K + N)
    q = _codes(rng, N, K)
    xq_h, xs_h = oracle.act_quant(wl.activations(62, M % 7, M, K))
    args = (torch.from_numpy(xq_h).to(DEV), dev_f32(xs_h), dev_packed(oracle.pack(q)),
            dev_f32([0.0173]))
    y = Guarded((M, N), torch.float32)
    acc = Guarded((M, N), torch.int32)
    _three_times(lambda: bl.bitlinear(*args, path=path, out=y.t, acc_out=acc.t), [y, acc])
    y0 = Guarded((M, N), torch.float32)
    _three_times(lambda: bl.bitlinear(*args, out=y0.t), [y0])
    assert torch.equal(y0.t.view(torch.int32), y.t.view(torch.int32))


@pytest.mark.parametrize("M,K,N", [(1, 64, 7), (1, 320, 200), (1, 4096, 33), (1, 4096, 2),
                                   (1, 8192, 31), (1, 8192, 3), (1, 16384, 1), (1, 20480, 17),
                                   (1, 28672, 9), (1, 32768, 5), (2, 320, 65)])
@pytest.mark.parametrize("norm", [False, True])
def test_quant_bitlinear_guards_and_repeats(M, K, N, norm):
    rng = np.random.default_rng(M + K + N + 7)
    x = dev_bf16(wl.activations(68, M, M, K))
    gain = dev_bf16(wl.rms_gain(68, 0, K)) if norm else None
    pk, g = dev_packed(oracle.pack(_codes(rng, N, K))), dev_f32([0.021])
    y, xq, xs = Guarded((M, N), torch.float32), Guarded((M, K), torch.int8), Guarded(M, torch.float32)
    _three_times(lambda: bl.quant_bitlinear(x, pk, g, rms_gain=gain, out=(y.t, xq.t, xs.t)),
                 [y, xq, xs])


def test_pair_and_other_formats_guards_and_repeats():
    M, K, N1, N2 = 4, 3200, 257, 1000
    rng = np.random.default_rng(63)
    xq_h, xs_h = oracle.act_quant(wl.activations(63, 0, M, K))
    xq, xs = torch.from_numpy(xq_h).to(DEV), dev_f32(xs_h)
    q1, q2 = _codes(rng, N1, K), _codes(rng, N2, K)
    g = dev_f32([0.02])
    y1, y2 = Guarded((M, N1), torch.float32), Guarded((M, N2), torch.float32)
    _three_times(lambda: bl.bitlinear_pair(xq, xs, dev_packed(oracle.pack(q1)), g,
                                           dev_packed(oracle.pack(q2)), g, out=(y1.t, y2.t)),
                 [y1, y2])
    W = dev_f32(wl.weights(63, 1, N1, K))
    bits, gb = bl.quantize_weights_binary(W)
    pk, gp = bl.quantize_weights(W)
    w3 = bl.pack_base3(pk, K)
    for fn, w, gg in ((bl.bitlinear_binary, bits, gb), (bl.bitlinear_base3, w3, gp)):
        y = Guarded((M, N1), torch.float32)
        acc = Guarded((M, N1), torch.int32)
        _three_times(lambda: fn(xq, xs, w, gg, out=y.t, acc_out=acc.t), [y, acc])


@pytest.mark.parametrize("K,N", [(64, 3), (8256, 9), (28672, 17)])
def test_one_token_formats_guards_and_repeats(K, N):
    rng = np.random.default_rng(K + N)
    xq_h, xs_h = oracle.act_quant(wl.activations(69, 0, 1, K))
    xq, xs = torch.from_numpy(xq_h).to(DEV), dev_f32(xs_h)
    qb = np.where(rng.random((N, K)) < 0.5, -1, 1).astype(np.int8)
    bits = torch.from_numpy(oracle.pack_binary(qb).view(np.int32)).to(DEV)
    q3 = _codes(rng, N, K)
    w3 = bl.pack_base3(dev_packed(oracle.pack(q3)), K)
    g = dev_f32([0.03])
    for fn, w in ((bl.bitlinear_binary, bits), (bl.bitlinear_base3, w3)):
        y = Guarded((1, N), torch.float32)
        acc = Guarded((1, N), torch.int32)
        _three_times(lambda: fn(xq, xs, w, g, out=y.t, acc_out=acc.t), [y, acc])


# ---------------------------------------------------------- glue, FFN ----

@pytest.mark.parametrize("kind", ["relu2", "swiglu"])
def test_glu_guards_and_repeats(kind):
    M, K = 5, 6848
    g, u = wl.ffn_hidden(64, 0, M, K)
    gd, ud = dev_f32(g), dev_f32(u)
    for count in (1, 3, M * K):
        h = Guarded(count, torch.bfloat16)
        _three_times(lambda: bl.glu(gd.view(-1)[:count], ud.view(-1)[:count], kind, out=h.t),
                     [h])
    gain = dev_bf16(wl.rms_gain(64, 1, K))
    for gn in (None, gain):
        hq, hs = Guarded((M, K), torch.int8), Guarded(M, torch.float32)
        _three_times(lambda: bl.glu_quant(gd, ud, kind, subln_gain=gn, out=(hq.t, hs.t)),
                     [hq, hs])


@pytest.mark.parametrize("M", [1, 4, 5, 16, 40])
def test_ffn_step_guards_and_repeats(M):
    K, N = 2560, 6912
    Ws = []
    for i, (n, k) in enumerate([(N, K), (N, K), (K, N)]):
        Ws += list(bl.quantize_weights(dev_f32(wl.weights(65, i, n, k))))
    x = dev_bf16(wl.activations(65, M, M, K))
    gain = dev_bf16(wl.rms_gain(65, 2, N))
    ws = Guarded(bl.lib().bl_ffn_relu2_workspace_bytes(M, K, N), torch.uint8)
    for kind, gn in (("relu2", None), ("relu2", gain), ("swiglu", None)):
        y = Guarded((M, K), torch.float32)
        _three_times(lambda: bl.ffn_step(x, *Ws, kind=kind, subln_gain=gn, workspace=ws.t,
                                         out=y.t), [y, ws])
        y2 = Guarded((M, K), torch.float32)
        _three_times(lambda: bl.ffn_step_noalloc(x, *Ws, kind=kind, subln_gain=gn, out=y2.t),
                     [y2])
        assert torch.equal(y.t.view(torch.int32), y2.t.view(torch.int32))


# ------------------------------------------------ straight-through backward ----

# The last two shapes' dW take more than one launch (273 tiles of 128 x 256):
# at 33 tokens the last two row tiles run as 64 x 64 tiles, at 512 tokens
# they split their 16 stages over two workgroups each, whose partial tiles
# sit in the workspace until a third launch adds them.
@pytest.mark.parametrize("M,N,K", [(3, 40, 128), (130, 264, 192), (257, 1000, 1344),
                                   (33, 2600, 3328), (512, 2600, 3328)])
def test_ste_guards_and_repeats(M, N, K):
    rng = np.random.default_rng(66 + M)
    q = _codes(rng, N, K)
    qT = bl.pack_ste_t(dev_packed(oracle.pack(q)), K)
    dy = dev_bf16(wl.f32_to_bf16_bits((rng.standard_normal((M, N)) * 0.01).astype(np.float32)))
    dx = Guarded((M, K), torch.float32)
    _three_times(lambda: bl.ste_backward_dx(dy, qT, dev_f32([0.02]), N, out=dx.t), [dx])
    xq_h, xs_h = oracle.act_quant(wl.activations(66, 1, M, K))
    ws = Guarded(bl.lib().bl_ste_dw_workspace_bytes(M, N, K), torch.uint8)
    dW = Guarded((N, K), torch.float32)
    _three_times(lambda: bl.ste_backward_dw(dy, torch.from_numpy(xq_h).to(DEV), dev_f32(xs_h),
                                            workspace=ws.t, out=dW.t), [dW, ws])
