"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs. Integer results (gamma, packed bytes, activation codes,
int32 sums) must be bit-exact; fp32 outputs within 1e-6 relative,
elementwise; fused-RMSNorm scales within 1e-6 relative."""
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
RTOL_Y = 1e-6
RTOL_SCALE_FUSED = 1e-6


# ------------------------------------------------------------- helpers ----

def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).to(DEV) \
        .view(torch.bfloat16)


def dev_packed(p):
    return torch.from_numpy(np.ascontiguousarray(p, np.uint32).view(np.int32)).to(DEV)


def host_packed(t):
    return t.cpu().numpy().view(np.uint32)


def gpu_weights(W):
    pk, g = bl.quantize_weights(dev_f32(W))
    return pk, g


def assert_y_close(y, y_ref, what=""):
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    bad = np.abs(y - y_ref) > RTOL_Y * np.abs(y_ref)
    assert not bad.any(), f"{what}: {bad.sum()} outputs beyond 1e-6 relative, e.g. " \
        f"{y[bad][:3]} vs {y_ref[bad][:3]}"


def rand_codes(rng, N, K):
    return rng.integers(-1, 2, size=(N, K)).astype(np.int8)


# ------------------------------------------------- weight quantisation ----

@pytest.mark.parametrize("N,K", [(1, 64), (7, 64), (16, 128), (200, 320), (33, 3200),
                                 (257, 8640), (64, 28672)])
def test_weight_quant_small(N, K):
    W = wl.weights(50, 0, N, K)
    pk_ref, g_ref, _ = oracle.quantize_weights(W)
    pk, g = gpu_weights(W)
    assert g.item() == float(g_ref)
    assert np.array_equal(host_packed(pk), pk_ref)


def test_weight_quant_forced_ties():
    rng = np.random.default_rng(51)
    W = (0.02 * rng.standard_normal((16, 64))).astype(np.float32)
    # Fixed point: W[3,5] = 0.5*(gamma+eps) with gamma of the final matrix.
    for _ in range(50):
        g = oracle.absmean_gamma(W)
        t = np.float32(0.5) * (np.float32(g) + np.float32(oracle.WEIGHT_EPS))
        if W[3, 5] == t and W[7, 9] == -t:
            break
        W[3, 5] = t
        W[7, 9] = -t
    else:
        raise AssertionError("tie construction did not converge")
    assert np.float32(W[3, 5]) / (np.float32(g) + np.float32(oracle.WEIGHT_EPS)) == 0.5
    pk_ref, g_ref, q_ref = oracle.quantize_weights(W)
    assert q_ref[3, 5] == 0 and q_ref[7, 9] == 0
    pk, g = gpu_weights(W)
    assert g.item() == float(g_ref)
    assert np.array_equal(host_packed(pk), pk_ref)


def test_weight_quant_zero_matrix():
    W = np.zeros((32, 128), np.float32)
    pk, g = gpu_weights(W)
    assert g.item() == 0.0
    assert (host_packed(pk) == 0x55555555).all()


_WCACHE = {}


def workload_weights(wid, idx):
    """(codes, gamma) from the oracle and (packed, gamma) from the GPU for one
    full-size workload matrix, after checking the two agree bit-exactly."""
    key = (wid, idx)
    if key not in _WCACHE:
        if len(_WCACHE) >= 2:
            _WCACHE.clear()
        _, K, N = wl.WORKLOADS[wid][1][idx]
        W = wl.weights(wid, idx, N, K)
        pk_ref, g_ref, q_ref = oracle.quantize_weights(W)
        pk, g = gpu_weights(W)
        del W
        assert g.item() == float(g_ref)
        assert np.array_equal(host_packed(pk), pk_ref)
        _WCACHE[key] = (q_ref, g_ref, pk, g)
    return _WCACHE[key]


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_weight_quant_workloads_full(wid):
    """Every weight matrix of every workload at full size: bit-exact."""
    for idx in range(len(wl.WORKLOADS[wid][1])):
        workload_weights(wid, idx)


# --------------------------------------------- activation quantisation ----

@pytest.mark.parametrize("M,K", [(1, 64), (3, 2560), (16, 3200), (300, 6912), (2, 28672)])
@pytest.mark.parametrize("fused", [False, True])
def test_act_quant(M, K, fused):
    x = wl.activations(52, 0, M, K)
    gain = wl.rms_gain(52, 0, K) if fused else None
    xq_ref, xs_ref = oracle.act_quant(x, gain)
    xq, xs = bl.quantize_acts(dev_bf16(x), None if gain is None else dev_bf16(gain))
    assert np.array_equal(xq.cpu().numpy(), xq_ref)
    xs = xs.cpu().numpy()
    if fused:
        assert np.all(np.abs(xs - xs_ref) <= RTOL_SCALE_FUSED * xs_ref)
    else:
        assert np.array_equal(xs, xs_ref)


def test_act_quant_golden_and_zero_token():
    import os
    cases = []
    path = os.path.join(os.path.dirname(__file__), "golden", "act_quant_ties.txt")
    cur = None
    for line in open(path):
        line = line.strip()
        if line.startswith("x:"):
            cur = [float(v) for v in line[2:].split()]
        elif line.startswith("codes:"):
            cases.append((cur, [int(v) for v in line[6:].split()]))
    K = 64
    x = np.zeros((len(cases) + 1, K), np.float32)   # last token all zero
    for i, (vals, _) in enumerate(cases):
        x[i, :len(vals)] = vals
    xb = wl.f32_to_bf16_bits(x)
    xq, xs = bl.quantize_acts(dev_bf16(xb))
    xq = xq.cpu().numpy()
    xs = xs.cpu().numpy()
    for i, (vals, codes) in enumerate(cases):
        assert xq[i, :len(codes)].tolist() == codes
        assert (xq[i, len(codes):] == 0).all()
    assert (xq[-1] == 0).all()
    assert xs[-1] == np.float32(1e-5) / np.float32(127)


# ------------------------------- act quant + product in one call ----

# One launch at one token with K <= 4096 (one or several row waves, RW = 1
# below four rows); the others take the two-call route.
# One launch: K <= 4096 (cached kernel), and without a gain whole pieces of
# 4096 up to 32768 (rows kernel at 2-4 pieces from N >= 4 or 2, else stream;
# ragged last waves and workgroups included). Two launches: a partial second
# piece (4160, 6912), nine pieces (36864), several tokens, and every long row
# with a gain.
QUANT_BITLINEAR_CASES = [
    (1, 64, 7), (1, 64, 1), (1, 320, 200), (1, 2560, 2560), (1, 3200, 8640), (1, 4096, 33),
    (1, 4096, 3), (1, 4160, 100), (1, 6912, 11), (1, 8192, 300), (1, 8192, 37), (1, 8192, 3),
    (1, 12288, 100), (1, 12288, 2), (1, 16384, 1), (1, 16384, 9), (1, 16384, 2),
    (1, 20480, 5), (1, 24576, 17), (1, 28672, 64), (1, 32768, 7), (1, 36864, 3),
    (3, 2560, 257),
]


@pytest.mark.parametrize("M,K,N", QUANT_BITLINEAR_CASES)
@pytest.mark.parametrize("norm", [False, True])
def test_quant_bitlinear(M, K, N, norm):
    """bl_quant_bitlinear: x_q and x_scale carry the bits of bl_quantize_acts,
    y the bits of bl_bitlinear on them; against the oracle the codes and the
    int32 sums are exact and y is within 1e-6."""
    rng = np.random.default_rng(M * 100003 + K + N)
    x = wl.activations(67, M, M, K)
    gain = wl.rms_gain(67, 1, K) if norm else None
    q = rand_codes(rng, N, K)
    pk, g = dev_packed(oracle.pack(q)), dev_f32([0.0131])
    xd = dev_bf16(x)
    gd = None if gain is None else dev_bf16(gain)
    y, xq, xs = bl.quant_bitlinear(xd, pk, g, rms_gain=gd)
    xq2, xs2 = bl.quantize_acts(xd, gd)
    y2, acc = bl.bitlinear(xq2, xs2, pk, g, return_acc=True)
    assert torch.equal(xq, xq2)
    assert torch.equal(xs.view(torch.int32), xs2.view(torch.int32))
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
    xq_ref, xs_ref = oracle.act_quant(x, gain)
    assert np.array_equal(xq.cpu().numpy(), xq_ref)
    xs_h = xs.cpu().numpy()
    if norm:
        assert np.all(np.abs(xs_h - xs_ref) <= RTOL_SCALE_FUSED * xs_ref)
    else:
        assert np.array_equal(xs_h, xs_ref)
    acc_ref = oracle.int_matmul(xq_ref, q)
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert_y_close(y.cpu().numpy(), oracle.epilogue(acc_ref, xs_ref, np.float32(0.0131)),
                   f"quant_bitlinear M={M} K={K} N={N}")


@pytest.mark.parametrize("K", [64, 4096, 8192, 16384, 28672, 32768])
def test_quant_bitlinear_golden_ties_and_zero_token(K):
    """The in-kernel quantiser on the golden tie tokens (each as its own
    one-token call, mirrored in sign too) and on an all-zero token: the golden
    codes, and the products of identity rows give codes times the scale."""
    toks, expect = [], []
    for vals, codes in _golden_act_cases():
        toks.append(vals)
        expect.append(codes)
        toks.append([vals[0]] + [-v for v in vals[1:]])
        expect.append([codes[0]] + [-c for c in codes[1:]])
    toks.append([0.0])
    expect.append([0])
    N = 64
    ident = dev_packed(oracle.pack(_select_codes(N, K, [(n,) for n in range(N)])))
    one = dev_f32([1.0])
    for vals, codes in zip(toks, expect):
        x = np.zeros((1, K), np.float32)
        x[0, :len(vals)] = vals
        xb = wl.f32_to_bf16_bits(x)
        y, xq, xs = bl.quant_bitlinear(dev_bf16(xb), ident, one)
        xq = xq.cpu().numpy()[0]
        assert xq[:len(codes)].tolist() == codes
        assert (xq[len(codes):] == 0).all()
        ref_q, ref_s = oracle.act_quant(xb)
        assert np.array_equal(xq, ref_q[0]) and xs.cpu().numpy()[0] == ref_s[0]
        y = y.cpu().numpy()[0]
        assert np.array_equal(y, (xq[:N].astype(np.float32) * ref_s[0]).astype(np.float32))
    assert ref_s[0] == np.float32(1e-5) / np.float32(127)


@pytest.mark.parametrize("K,N", [(8192, 28672), (28672, 8192)])
def test_quant_bitlinear_70b_rows(K, N):
    """bl_quant_bitlinear at the full 70B-class decode shapes (one launch): the
    codes and the scale are the oracle's bits, and every output is within
    1e-6 of the oracle's epilogue of its exact int32 product (an int32 sum
    off by one would move y by 1/|sum|, far more at these sums)."""
    rng = np.random.default_rng(K + 7 * N)
    x = wl.activations(71, 0, 1, K)
    q = rand_codes(rng, N, K)
    gm = np.float32(0.0173)
    y, xq, xs = bl.quant_bitlinear(dev_bf16(x), dev_packed(oracle.pack(q)), dev_f32([gm]))
    xq_ref, xs_ref = oracle.act_quant(x)
    assert np.array_equal(xq.cpu().numpy(), xq_ref)
    assert np.array_equal(xs.cpu().numpy(), xs_ref)
    acc_ref = oracle.int_matmul(xq_ref, q)
    assert_y_close(y.cpu().numpy(), oracle.epilogue(acc_ref, xs_ref, gm), f"70B rows K={K} N={N}")


# ------------------------------------------------------------ product ----

def _product_case(M, K, N, seed):
    rng = np.random.default_rng(seed)
    q = rand_codes(rng, N, K)
    # Skewed codes: a few all-(+1) / all-(-1) / all-zero rows.
    if N > 3:
        q[0] = 1
        q[1] = -1
        q[2] = 0
    x = wl.activations(seed, 0, M, K)
    xq, xs = oracle.act_quant(x)
    if M > 1:
        xq[-1] = 127   # extreme token: |acc| up to 127*K
    g = np.float32(0.0159)
    return q, xq, xs, g


GEMV_CASES = [(1, 64, 1), (1, 320, 200), (2, 3200, 50), (5, 8640, 33), (16, 6912, 257),
              (16, 2560, 16), (1, 28672, 40), (3, 1024, 4),
              # two row groups per workgroup (>= 8 tokens, >= 384 groups), the
              # last workgroup's second group partly / wholly past N
              (12, 2560, 6200), (9, 1024, 6150)]
GEMM_CASES = [(1, 64, 1), (17, 320, 200), (64, 3200, 50), (100, 2560, 300), (300, 8640, 129),
              (513, 640, 260), (256, 256, 256), (70, 28672, 65)]


@pytest.mark.parametrize("M,K,N", GEMV_CASES)
def test_gemv_parity(M, K, N):
    q, xq, xs, g = _product_case(M, K, N, 53)
    y_ref, acc_ref = oracle.bitlinear(xq, xs, q, g)
    y, acc = bl.bitlinear(torch.from_numpy(xq).to(DEV), dev_f32(xs), dev_packed(oracle.pack(q)),
                          dev_f32([g]), return_acc=True, path=1)
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert_y_close(y.cpu().numpy(), y_ref, "gemv")


# One-token GEMV (path 4): K <= 4096 and <= 8192 run the register-cached
# variant (one or two 1 KB pieces per row, four / two rows per wave, one row
# when N is smaller), longer rows the LDS-streamed one (one row per wave);
# K = 4160 / 8256 / 2560 / 6912 end in a partial piece, K = 65536 stages
# more activation slots than a thread holds across the weight issue.
# Every launch shape of the one-token GEMV: one piece (four rows or one row
# per wave), two pieces (partial, whole), three to eight whole pieces, and a
# partial last piece past two.
ONE_TOKEN_CASES = [(64, 1), (320, 200), (4096, 3), (4096, 4), (2560, 6912), (4160, 1),
                   (4160, 7), (8192, 2049), (8192, 1), (8192, 5), (6912, 2560), (8256, 33),
                   (12288, 1), (12288, 7), (16384, 17), (16384, 1), (20480, 9), (24576, 3),
                   (28672, 40), (28672, 8193), (32768, 15), (65536, 5), (3200, 3203),
                   (11008, 100)]


@pytest.mark.parametrize("K,N", ONE_TOKEN_CASES)
def test_one_token_gemv_parity(K, N):
    """Path 4 against the oracle: int32 sums bit-exact, outputs within 1e-6,
    and the automatic choice gives the same bits. The token is the extreme
    +127 row, then one with the full int8 range (-128 included), so the
    masked-field sums and the activation-sum correction run at their largest."""
    q, xq, xs, g = _product_case(1, K, N, 57)
    rng = np.random.default_rng(K + N)
    tokens = [np.full((1, K), 127, np.int8), rng.integers(-128, 128, (1, K)).astype(np.int8),
              xq]
    args_w = (dev_packed(oracle.pack(q)), dev_f32([g]))
    for t in tokens:
        y_ref, acc_ref = oracle.bitlinear(t, xs, q, g)
        xt = torch.from_numpy(t).to(DEV)
        y, acc = bl.bitlinear(xt, dev_f32(xs), *args_w, return_acc=True, path=4)
        assert np.array_equal(acc.cpu().numpy(), acc_ref)
        assert_y_close(y.cpu().numpy(), y_ref, "one-token gemv")
        y0 = bl.bitlinear(xt, dev_f32(xs), *args_w)
        assert torch.equal(y0.view(torch.int32), y.view(torch.int32))


def test_one_token_gemv_rejects_other_shapes():
    q, xq, xs, g = _product_case(2, 128, 8, 58)
    args = (dev_packed(oracle.pack(q)), dev_f32([g]))
    with pytest.raises(bl.BitLinearError):
        bl.bitlinear(torch.from_numpy(xq).to(DEV), dev_f32(xs), *args, path=4)
    q, xq, xs, g = _product_case(1, 65600, 2, 58)
    with pytest.raises(bl.BitLinearError):
        bl.bitlinear(torch.from_numpy(xq).to(DEV), dev_f32(xs), dev_packed(oracle.pack(q)),
                     dev_f32([g]), path=4)


@pytest.mark.parametrize("M,K,N", GEMM_CASES)
def test_gemm_parity(M, K, N):
    q, xq, xs, g = _product_case(M, K, N, 54)
    y_ref, acc_ref = oracle.bitlinear(xq, xs, q, g)
    y, acc = bl.bitlinear(torch.from_numpy(xq).to(DEV), dev_f32(xs), dev_packed(oracle.pack(q)),
                          dev_f32([g]), return_acc=True, path=2)
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert_y_close(y.cpu().numpy(), y_ref, "gemm")


# Large grids select the large prefill tiles: 128 x 256 with two workgroups
# per CU for the first shape, 128 x 512 with one for the next three (the
# fourth with only 160 tiles), and 128 x 320 tiles of 10 waves (activation
# loads dealt unevenly over the waves) for the last two, whose N is a
# multiple of 320; the shapes are ragged in M (and N for the first four),
# and K = 320 / 192 / 2624 / 704 ends in a half (64-deep) K step.
LARGE_TILE_CASES = [(2000, 320, 4000), (2000, 192, 8000), (2048, 384, 8192), (1935, 448, 5000),
                    (4000, 2624, 2560), (4050, 704, 1920)]


@pytest.mark.parametrize("M,K,N", LARGE_TILE_CASES)
def test_gemm_large_tiles_ragged(M, K, N):
    q, xq, xs, g = _product_case(M, K, N, 58)
    y, acc = bl.bitlinear(torch.from_numpy(xq).to(DEV), dev_f32(xs), dev_packed(oracle.pack(q)),
                          dev_f32([g]), return_acc=True, path=2)
    # Every int32 sum: an fp64 product of the integer operands is exact here
    # (|acc| <= 127 * K < 2^53).
    ref64 = torch.from_numpy(xq).to(DEV, torch.float64) @ torch.from_numpy(q).to(
        DEV, torch.float64).t().contiguous()
    assert torch.equal(acc.to(torch.float64), ref64)
    # Oracle on a sample of tokens (first, last and every row-tile edge), all
    # output features.
    rng = np.random.default_rng(M + N)
    edges = [m for t in range(0, M, 128) for m in (t, min(t + 127, M - 1))]
    ms = np.unique(np.concatenate([rng.choice(M, 8, replace=False), edges[:6], edges[-6:]]))
    y_ref, acc_ref = oracle.bitlinear(xq[ms], xs[ms], q, g)
    idx = torch.from_numpy(ms).to(DEV)
    assert np.array_equal(acc[idx].cpu().numpy(), acc_ref)
    assert_y_close(y[idx].cpu().numpy(), y_ref, "gemm large tiles")
    sc = (dev_f32(xs) * dev_f32([g])).view(-1, 1)
    assert torch.equal(y, acc.to(torch.float32) * sc)


# Few tiles split K across workgroups whose int32 partial sums are added into
# y; y starts with garbage here (NaN bits) to show it is cleared first. With
# many steps per split the workgroups also hold K groups: four for the
# 80-token case on K near 28672, two (4-deep ring) for the 64-token one and
# two for the 100-token one; the last two
# end K in a half step, and their last split's step count is not a multiple
# of the group count.
SPLIT_K_CASES = [(64, 8192, 700), (64, 28672, 260), (33, 6912, 1000), (80, 28672, 8192),
                 (100, 2560, 300), (300, 8640, 129), (64, 28352, 8100), (100, 24384, 2000)]


@pytest.mark.parametrize("M,K,N", SPLIT_K_CASES)
def test_gemm_split_k(M, K, N):
    q, xq, xs, g = _product_case(M, K, N, 59)
    args = (torch.from_numpy(xq).to(DEV), dev_f32(xs), dev_packed(oracle.pack(q)), dev_f32([g]))
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    acc = torch.full((M, N), -7, dtype=torch.int32, device=DEV)
    for _ in range(2):
        bl.bitlinear(*args, out=y, acc_out=acc, path=2)
        ref64 = args[0].to(torch.float64) @ torch.from_numpy(q).to(DEV, torch.float64).t().contiguous()
        assert torch.equal(acc.to(torch.float64), ref64)
        sc = (args[1] * args[3]).view(-1, 1)
        assert torch.equal(y, acc.to(torch.float32) * sc)
    rng = np.random.default_rng(M * N)
    ms = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, 6), replace=False)]))
    y_ref, acc_ref = oracle.bitlinear(xq[ms], xs[ms], q, g)
    idx = torch.from_numpy(ms).to(DEV)
    assert np.array_equal(acc[idx].cpu().numpy(), acc_ref)
    assert_y_close(y[idx].cpu().numpy(), y_ref, "split-K gemm")


# Few tiles but many tokens: two K groups inside each workgroup (with a
# 4-deep ring for long K with at most one tile per CU) add their partial
# sums through LDS.
# Step counts are not multiples of the group count, so some group's last step
# lies past K (its weights expand as zeros); the last three cases end K in a
# half (64-deep) step; M and N are ragged. y starts as NaN bits.
K_GROUP_CASES = [(512, 3200, 3200),   # 200 tiles of 64 x 128, 25 steps: two groups
                 (260, 2624, 6900),   # 270 tiles, 21 steps: two groups
                 (500, 8512, 3160),   # 200 tiles, 66.5 steps: 4-deep ring
                 (130, 6976, 8190),   # 192 tiles, 54.5 steps: 4-deep ring
                 # At most 64 tokens: two groups with a 4-deep ring (193
                 # tiles, 48.5 steps, ragged N), or 64 x 64 tiles with four
                 # groups instead of a split (128 tiles of 32 whole steps; 135
                 # tiles of 24.5 steps with ragged N)
                 (48, 6208, 24600), (50, 4096, 8192), (64, 3136, 8620),
                 # N a multiple of 160 where 128 x 128 tiles would spill
                 # into a second round: 128 x 160 tiles of two groups (216
                 # tiles, 24.5 steps; 208 tiles of 24 whole steps)
                 (500, 3136, 8640), (450, 3072, 8320)]


@pytest.mark.parametrize("M,K,N", K_GROUP_CASES)
def test_gemm_k_groups(M, K, N):
    q, xq, xs, g = _product_case(M, K, N, 61)
    args = (torch.from_numpy(xq).to(DEV), dev_f32(xs), dev_packed(oracle.pack(q)), dev_f32([g]))
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    acc = torch.full((M, N), -7, dtype=torch.int32, device=DEV)
    ref64 = args[0].to(torch.float64) @ torch.from_numpy(q).to(DEV, torch.float64).t().contiguous()
    for _ in range(2):
        bl.bitlinear(*args, out=y, acc_out=acc, path=2)
        assert torch.equal(acc.to(torch.float64), ref64)
        sc = (args[1] * args[3]).view(-1, 1)
        assert torch.equal(y, acc.to(torch.float32) * sc)
    rng = np.random.default_rng(M * N + 1)
    edges = [m for t in range(0, M, 64) for m in (t, min(t + 63, M - 1))]
    ms = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 6, replace=False), edges[-4:]]))
    y_ref, acc_ref = oracle.bitlinear(xq[ms], xs[ms], q, g)
    idx = torch.from_numpy(ms).to(DEV)
    assert np.array_equal(acc[idx].cpu().numpy(), acc_ref)
    assert_y_close(y[idx].cpu().numpy(), y_ref, "k-group gemm")


# The wide GEMV (17..64 tokens, 128 rows per workgroup, K in 512 blocks):
# K tails of half a block and half a chunk, ragged N, and the split-K path.
WIDE_CASES = [(17, 320, 200), (33, 2560, 300), (64, 8192, 700), (64, 6912, 1000),
              (48, 8640, 257), (64, 28672, 130), (20, 64, 5), (40, 1024, 4000)]


@pytest.mark.parametrize("M,K,N", WIDE_CASES)
def test_wide_gemv_parity(M, K, N):
    q, xq, xs, g = _product_case(M, K, N, 60)
    args = (torch.from_numpy(xq).to(DEV), dev_f32(xs), dev_packed(oracle.pack(q)), dev_f32([g]))
    y, acc = bl.bitlinear(*args, return_acc=True, path=3)
    y_ref, acc_ref = oracle.bitlinear(xq, xs, q, g)
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert_y_close(y.cpu().numpy(), y_ref, "wide gemv")
    y2, acc2 = bl.bitlinear(*args, return_acc=True, path=2)
    assert torch.equal(acc, acc2) and torch.equal(y.view(torch.int32), y2.view(torch.int32))


@pytest.mark.parametrize("M,K,N", [(37, 9216, 12777), (64, 28672, 8192)])
def test_wide_gemv_multi_block_splits_sampled(M, K, N):
    """Wide GEMV where each split streams several K blocks (the first shape's
    last split is short), on a sample of output features by the oracle."""
    q, xq, xs, g = _product_case(M, K, N, 61)
    args = (torch.from_numpy(xq).to(DEV), dev_f32(xs), dev_packed(oracle.pack(q)), dev_f32([g]))
    y, acc = bl.bitlinear(*args, return_acc=True, path=3)
    rng = np.random.default_rng(M + N)
    ns = np.unique(np.concatenate([rng.choice(N, 256, replace=False), [0, 1, 2, N - 1]]))
    y_ref, acc_ref = oracle.bitlinear(xq, xs, q[ns], g)
    nsd = torch.from_numpy(ns).to(DEV)
    assert np.array_equal(acc[:, nsd].cpu().numpy(), acc_ref)
    assert_y_close(y[:, nsd].cpu().numpy(), y_ref, "wide gemv multi-block")
    assert torch.equal(y, acc.to(torch.float32) * (dev_f32(xs) * dev_f32([g])).view(-1, 1))
    y0 = bl.bitlinear(*args)            # automatic choice: same bits
    assert torch.equal(y0.view(torch.int32), y.view(torch.int32))


def _random_shapes(n, seed, budget=1.5e8):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 17, 31, 33, 47, 64, 65, 100, 129, 257]))
        K = 64 * int(rng.integers(1, 97))
        N = int(rng.integers(1, 3001))
        if M * N * K <= budget:
            out.append((M, K, N))
    return out


@pytest.mark.parametrize("M,K,N", _random_shapes(24, 1234))
def test_random_shapes_every_path(M, K, N):
    """Seeded random shapes through every product path that applies
    (automatic, GEMV, GEMM, wide GEMV, one-token GEMV): int32 sums equal to the oracle's,
    outputs within 1e-6."""
    q, xq, xs, g = _product_case(M, K, N, 70 + M + K + N)
    y_ref, acc_ref = oracle.bitlinear(xq, xs, q, g)
    args = (torch.from_numpy(xq).to(DEV), dev_f32(xs), dev_packed(oracle.pack(q)), dev_f32([g]))
    paths = [0, 2]
    if M <= 16 and M * K <= 128 * 1024:
        paths.append(1)
    if M == 1 and K <= 65536:
        paths.append(4)
    if M <= 64:
        paths.append(3)
    for path in paths:
        y, acc = bl.bitlinear(*args, return_acc=True, path=path)
        assert np.array_equal(acc.cpu().numpy(), acc_ref), f"path {path}"
        assert_y_close(y.cpu().numpy(), y_ref, f"path {path}")


def test_gemv_and_gemm_agree_bitwise():
    for M, K, N in [(1, 2560, 6912), (16, 6912, 2560), (4, 3200, 8640)]:
        q, xq, xs, g = _product_case(M, K, N, 55)
        args = (torch.from_numpy(xq).to(DEV), dev_f32(xs), dev_packed(oracle.pack(q)),
                dev_f32([g]))
        y1, a1 = bl.bitlinear(*args, return_acc=True, path=1)
        y2, a2 = bl.bitlinear(*args, return_acc=True, path=2)
        y0 = bl.bitlinear(*args, path=0)
        assert torch.equal(a1, a2)
        assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
        assert torch.equal(y0.view(torch.int32), y1.view(torch.int32))


def test_determinism_repeated_calls():
    q, xq, xs, g = _product_case(300, 2560, 1000, 56)
    args = (torch.from_numpy(xq).to(DEV), dev_f32(xs), dev_packed(oracle.pack(q)), dev_f32([g]))
    outs = [bl.bitlinear(*args, path=p).view(torch.int32).clone() for p in (2, 2, 2)]
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    outs = [bl.bitlinear(args[0][:8].contiguous(), args[1][:8].contiguous(), args[2], args[3],
                         path=1).view(torch.int32).clone() for _ in range(3)]
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    outs = [bl.bitlinear(args[0][:1].contiguous(), args[1][:1].contiguous(), args[2], args[3],
                         path=4).view(torch.int32).clone() for _ in range(3)]
    assert all(torch.equal(outs[0], o) for o in outs[1:])


def test_zero_weights_give_zero_output():
    W = np.zeros((48, 256), np.float32)
    pk, g = gpu_weights(W)
    x = wl.activations(57, 0, 20, 256)
    xq, xs = bl.quantize_acts(dev_bf16(x))
    for path in (1, 2):
        xin = xq[:4].contiguous() if path == 1 else xq
        sin = xs[:4].contiguous() if path == 1 else xs
        y, acc = bl.bitlinear(xin, sin, pk, g, return_acc=True, path=path)
        assert int(acc.abs().max()) == 0 and float(y.abs().max()) == 0.0


# --------------------------------------------- full workloads (sampled) ----

def _workload_cases():
    out = []
    for wid, (_, projs, Ms) in wl.WORKLOADS.items():
        for idx, (name, K, N) in enumerate(projs):
            for M in Ms:
                out.append((wid, idx, name, K, N, M))
    return out


@pytest.mark.parametrize("wid,idx,name,K,N,M", _workload_cases(),
                         ids=lambda v: str(v))
def test_workload_full_size(wid, idx, name, K, N, M):
    """Full-size shapes in the benchmark's launch configuration: packed weights,
    gamma and activation codes compared in full; every int32 sum against an
    fp64 matrix product of the oracle's codes (exact: products and partial
    sums are integers below 2^53 in any order) and every output within 1e-6
    of the oracle's epilogue of those sums; a sample of tokens x features
    also through the oracle's own integer product."""
    fused = wid == 4
    q_ref, g_ref, pk, g = workload_weights(wid, idx)
    x = wl.activations(wid, idx, M, K)
    gain = wl.rms_gain(wid, idx, K) if fused else None
    xq_ref, xs_ref = oracle.act_quant(x, gain)
    xq, xs = bl.quantize_acts(dev_bf16(x), None if gain is None else dev_bf16(gain))
    assert np.array_equal(xq.cpu().numpy(), xq_ref)
    xs_h = xs.cpu().numpy()
    if fused:
        assert np.all(np.abs(xs_h - xs_ref) <= RTOL_SCALE_FUSED * xs_ref)
    else:
        assert np.array_equal(xs_h, xs_ref)
    y, acc = bl.bitlinear(xq, xs, pk, g, return_acc=True)
    acc_h = acc.cpu().numpy()
    acc_full = xq_ref.astype(np.float64) @ q_ref.astype(np.float64).T
    assert np.array_equal(acc_h, acc_full.astype(np.int32)), f"workload {wid} {name} M={M}"
    del acc_full
    assert_y_close(y.cpu().numpy(), oracle.epilogue(acc_h, xs_h, g_ref), f"workload {wid} {name}")
    rng = np.random.default_rng(1000 * wid + M)
    ms = np.arange(M) if M <= 16 else np.sort(rng.choice(M, 16, replace=False))
    ns = np.sort(rng.choice(N, min(N, 384), replace=False))
    ns = np.unique(np.concatenate([ns, [0, N - 1]]))
    y_ref, acc_ref = oracle.bitlinear(xq_ref[ms], xs_h[ms], q_ref[ns], g_ref)
    acc_s = acc[torch.from_numpy(ms).to(DEV)][:, torch.from_numpy(ns).to(DEV)].cpu().numpy()
    y_s = y[torch.from_numpy(ms).to(DEV)][:, torch.from_numpy(ns).to(DEV)].cpu().numpy()
    assert np.array_equal(acc_s, acc_ref)
    assert_y_close(y_s, y_ref, f"workload {wid} {name} M={M}")
    # Whole-output property: y is exactly the fp32 rescale of acc.
    sc = (xs * g).view(-1, 1)
    assert torch.equal(y, acc.to(torch.float32) * sc)


# ------------------------------------------------------------- blocks ----

@pytest.mark.parametrize("M", [1, 4, 16])
def test_ffn_block_2b4t_stagewise(M):
    """2B4T-shaped FFN: gate/up BitLinears, squared-ReLU gating, down BitLinear.
    Each stage is checked bit-exactly against the oracle run on the GPU's own
    output of the previous stage."""
    wid = 2
    _, projs, _ = wl.WORKLOADS[wid]
    Ws = {name: wl.weights(wid, i, N, K) for i, (name, K, N) in enumerate(projs)}
    ref = {name: oracle.quantize_weights(W) for name, W in Ws.items()}
    dev = {name: gpu_weights(W) for name, W in Ws.items()}
    x = wl.activations(wid, 9, M, 2560)
    xq, xs = bl.quantize_acts(dev_bf16(x))
    xq_ref, xs_ref = oracle.act_quant(x)
    assert np.array_equal(xq.cpu().numpy(), xq_ref)
    outs = {}
    for name in ("gate", "up"):
        y, acc = bl.bitlinear(xq, xs, dev[name][0], dev[name][1], return_acc=True)
        y_ref, acc_ref = oracle.bitlinear(xq_ref, xs_ref, ref[name][2], ref[name][1])
        assert np.array_equal(acc.cpu().numpy(), acc_ref)
        assert_y_close(y.cpu().numpy(), y_ref, name)
        outs[name] = y
    h = bl.relu2_glu(outs["gate"], outs["up"])
    h_ref = oracle.relu2_glu(outs["gate"].cpu().numpy(), outs["up"].cpu().numpy())
    assert np.array_equal(h.view(torch.int16).cpu().numpy().view(np.uint16), h_ref)
    hq, hs = bl.quantize_acts(h)
    hq_ref, hs_ref = oracle.act_quant(h_ref)
    assert np.array_equal(hq.cpu().numpy(), hq_ref)
    assert np.array_equal(hs.cpu().numpy(), hs_ref)
    y, acc = bl.bitlinear(hq, hs, dev["down"][0], dev["down"][1], return_acc=True)
    y_ref, acc_ref = oracle.bitlinear(hq_ref, hs_ref, ref["down"][2], ref["down"][1])
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert_y_close(y.cpu().numpy(), y_ref, "down")


def _ffn_workspace_offsets(M, K, N):
    """Segment offsets of the FFN step's workspace (h first, then the codes and
    scales of the unfused sequence), as the library lays it out; the tests
    read the step's intermediate h (and at 16 tokens its codes) from it."""
    a = lambda v: (v + 255) // 256 * 256
    off, o = {}, 0
    for name, size in (("h", 2 * M * N), ("xq", M * K), ("xs", 4 * M), ("yg", 4 * M * N),
                       ("yu", 4 * M * N), ("hq", M * N), ("hs", 4 * M)):
        off[name] = o
        o += a(size)
    return off


def _ws_h(ws, M, N):
    return ws[:2 * M * N].cpu().numpy().view(np.uint16).reshape(M, N)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_ffn_fused_step_against_oracle_2b4t(M):
    """The fused step (bl_ffn_relu2, two launches at 1 and 4 tokens, three at
    16) on the 2B4T shapes and the inputs of the stage-wise block test: its h
    (left in the workspace) and y equal the separate GPU calls bit for bit,
    and every stage of those equals the oracle run on the previous stage's
    GPU output (codes, int32 sums and h bit-exact, fp32 within 1e-6). End to
    end (the oracle alone from x), the h codes that flip are counted: a flip
    needs an fp32 gate/up output within an ulp of a bf16 rounding boundary."""
    wid = 2
    _, projs, _ = wl.WORKLOADS[wid]
    Ws = {name: wl.weights(wid, i, N, K) for i, (name, K, N) in enumerate(projs)}
    ref = {name: oracle.quantize_weights(W) for name, W in Ws.items()}
    dev = {name: gpu_weights(W) for name, W in Ws.items()}
    K, N = 2560, 6912
    xb = wl.activations(wid, 9, M, K)
    x = dev_bf16(xb)
    ws = bl.ffn_relu2_workspace(M, K, N, DEV)
    y = bl.ffn_relu2(x, *dev["gate"], *dev["up"], *dev["down"], workspace=ws)
    torch.cuda.synchronize()
    h_fused = _ws_h(ws, M, N).copy()
    # The separate calls.
    xq, xs = bl.quantize_acts(x)
    yg, acc_g = bl.bitlinear(xq, xs, *dev["gate"], return_acc=True)
    yu, acc_u = bl.bitlinear(xq, xs, *dev["up"], return_acc=True)
    h = bl.relu2_glu(yg, yu)
    hq, hs = bl.quantize_acts(h)
    y_sep, acc_d = bl.bitlinear(hq, hs, *dev["down"], return_acc=True)
    h_bits = h.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(h_fused, h_bits)
    assert torch.equal(y.view(torch.int32), y_sep.view(torch.int32))
    # Stage by stage against the oracle.
    xq_ref, xs_ref = oracle.act_quant(xb)
    assert np.array_equal(xq.cpu().numpy(), xq_ref) and np.array_equal(xs.cpu().numpy(), xs_ref)
    for name, yy, aa in (("gate", yg, acc_g), ("up", yu, acc_u)):
        y_ref, a_ref = oracle.bitlinear(xq_ref, xs_ref, ref[name][2], ref[name][1])
        assert np.array_equal(aa.cpu().numpy(), a_ref), name
        assert_y_close(yy.cpu().numpy(), y_ref, name)
    assert np.array_equal(h_bits, oracle.relu2_glu(yg.cpu().numpy(), yu.cpu().numpy()))
    hq_ref, hs_ref = oracle.act_quant(h_bits)
    assert np.array_equal(hq.cpu().numpy(), hq_ref) and np.array_equal(hs.cpu().numpy(), hs_ref)
    yd_ref, ad_ref = oracle.bitlinear(hq_ref, hs_ref, ref["down"][2], ref["down"][1])
    assert np.array_equal(acc_d.cpu().numpy(), ad_ref)
    assert_y_close(y.cpu().numpy(), yd_ref, "down")
    # End to end from x alone.
    yg_o = oracle.bitlinear(xq_ref, xs_ref, ref["gate"][2], ref["gate"][1])[0]
    yu_o = oracle.bitlinear(xq_ref, xs_ref, ref["up"][2], ref["up"][1])[0]
    h_o = oracle.relu2_glu(yg_o, yu_o)
    hq_o, hs_o = oracle.act_quant(h_o)
    h_flips = int((h_o != h_bits).sum())
    code_flips = int((hq_o != hq.cpu().numpy()).sum())
    assert h_flips <= max(4, h_o.size // 10000) and code_flips <= h_flips, (h_flips, code_flips)
    if code_flips == 0 and np.array_equal(hs_o, hs.cpu().numpy()):
        y_o = oracle.bitlinear(hq_o, hs_o, ref["down"][2], ref["down"][1])[0]
        assert_y_close(y.cpu().numpy(), y_o, "end to end")


def _golden_act_cases():
    import os
    cases = []
    path = os.path.join(os.path.dirname(__file__), "golden", "act_quant_ties.txt")
    cur = None
    for line in open(path):
        line = line.strip()
        if line.startswith("x:"):
            cur = [float(v) for v in line[2:].split()]
        elif line.startswith("codes:"):
            cases.append((cur, [int(v) for v in line[6:].split()]))
    return cases


def _select_codes(N, K, cols):
    """Ternary codes [N][K]: row n is +1 at the columns cols[n] (a tuple), 0 elsewhere."""
    q = np.zeros((N, K), np.int8)
    for n, cs in enumerate(cols):
        for c in cs:
            q[n, c] = 1
    return q


@pytest.mark.parametrize("M", [1, 4, 16])
def test_ffn_fused_quantisers_on_golden_ties(M):
    """The per-workgroup quantisers of the fused FFN step on tie values.
    Tokens: the golden tie tokens and their sign-mirrored copies (absmax 127
    or 254 in column 0, repeated in column 20). Gate rows all read column 0
    with gamma 1/127, so relu(gate)^2 is the token scale squared (a power of
    two) within an ulp. Launch A: up rows are the identity, so the h left in
    the workspace is the codes times a power of two and must give the golden
    codes. Launch B (the act quant of h): up row 0 adds columns 0 and 20 (254,
    h's absmax), the others one or two golden columns, so h's codes are
    (c_a + c_b) / 2 rounded half to even; the down rows are the identity, so
    y / y[0] * 127 gives them."""
    K, N = 2560, 6912
    toks, expect = [], []
    for vals, codes in _golden_act_cases():
        toks.append(vals)
        expect.append(codes)
        toks.append([vals[0]] + [-v for v in vals[1:]])
        expect.append([codes[0]] + [-c for c in codes[1:]])
    x = np.zeros((M, K), np.float32)
    exp_codes = np.zeros((M, K), np.int64)
    for m in range(M):
        t = m % len(toks)
        x[m, :len(toks[t])] = toks[t]
        x[m, 20] = toks[t][0]
        exp_codes[m, :len(expect[t])] = expect[t]
        exp_codes[m, 20] = 127
    xb = wl.f32_to_bf16_bits(x)
    assert np.array_equal(oracle.act_quant(xb)[0], exp_codes)
    gate = _select_codes(N, K, [(0,)] * N)
    up_id = _select_codes(N, K, [(n,) if n < K else () for n in range(N)])
    down_id = _select_codes(K, N, [(k,) for k in range(K)])
    g127 = np.float32(1.0) / np.float32(127.0)

    def run(up, ws):
        return bl.ffn_relu2(dev_bf16(xb), dev_packed(oracle.pack(gate)), dev_f32([g127]),
                            dev_packed(oracle.pack(up)), dev_f32([1.0]),
                            dev_packed(oracle.pack(down_id)), dev_f32([1.0]), workspace=ws)

    ws = bl.ffn_relu2_workspace(M, K, N, DEV)
    run(up_id, ws)
    torch.cuda.synchronize()
    h = wl.bf16_bits_to_f32(_ws_h(ws, M, N)).astype(np.float64)
    assert np.array_equal(np.rint(h[:, :K] * 127.0 / h[:, :1]).astype(np.int64), exp_codes)
    assert (h[:, K:] == 0).all()
    # Launch B.
    rng = np.random.default_rng(59)
    cols = list(range(10)) + [20]
    pairs = [(0, 20)]
    for _ in range(K - 1):
        a, b = rng.choice(cols, 2, replace=False)
        pairs.append((int(a),) if rng.random() < 0.2 else (int(a), int(b)))
    y = run(_select_codes(N, K, pairs + [()] * (N - K)), ws).cpu().numpy().astype(np.float64)
    hv = np.stack([exp_codes[:, list(p)].sum(axis=1) for p in pairs], axis=1).astype(np.float64)
    assert (np.abs(hv).max(axis=1) == 254).all()
    want = np.rint(hv / 2.0)  # half to even
    assert (np.abs(hv / 2.0 - np.floor(hv / 2.0)) == 0.5).any()  # ties present
    assert np.array_equal(np.rint(y * 127.0 / y[:, :1]), want)


@pytest.mark.parametrize("M", [1, 512])
def test_block_3b_stagewise(M):
    """3B-class block linear set: fused RMSNorm + quant feeding q/k/v (shared
    input), o, gate/up (shared input) and down."""
    wid = 4
    _, projs, _ = wl.WORKLOADS[wid]
    inputs = {"qkv": (10, 3200), "o": (11, 3200), "gu": (12, 3200), "down": (13, 8640)}
    users = {"q": "qkv", "k": "qkv", "v": "qkv", "o": "o", "gate": "gu", "up": "gu",
             "down": "down"}
    quant = {}
    for key, (ix, K) in inputs.items():
        x = wl.activations(wid, ix, M, K)
        gain = wl.rms_gain(wid, ix, K)
        xq, xs = bl.quantize_acts(dev_bf16(x), dev_bf16(gain))
        xq_ref, xs_ref = oracle.act_quant(x, gain)
        assert np.array_equal(xq.cpu().numpy(), xq_ref), key
        assert np.all(np.abs(xs.cpu().numpy() - xs_ref) <= RTOL_SCALE_FUSED * xs_ref), key
        quant[key] = (xq, xs, xq_ref)
    rng = np.random.default_rng(58)
    for i, (name, K, N) in enumerate(projs):
        W = wl.weights(wid, i, N, K)
        pk_ref, g_ref, q_ref = oracle.quantize_weights(W)
        pk, g = gpu_weights(W)
        assert np.array_equal(host_packed(pk), pk_ref) and g.item() == float(g_ref)
        xq, xs, xq_ref = quant[users[name]]
        y, acc = bl.bitlinear(xq, xs, pk, g, return_acc=True)
        ms = np.arange(M) if M <= 16 else np.sort(rng.choice(M, 24, replace=False))
        y_ref, acc_ref = oracle.bitlinear(xq_ref[ms], xs.cpu().numpy()[ms], q_ref, g_ref)
        assert np.array_equal(acc.cpu().numpy()[ms], acc_ref), name
        assert_y_close(y.cpu().numpy()[ms], y_ref, name)


# ---------------------------------------------------------------- glue ----

def test_relu2_glu_parity():
    g, u = wl.ffn_hidden(59, 0, 7, 1001)
    h = bl.relu2_glu(dev_f32(g), dev_f32(u))
    assert np.array_equal(h.view(torch.int16).cpu().numpy().view(np.uint16),
                          oracle.relu2_glu(g, u))
    for count in (1, 3, 5):
        h = bl.relu2_glu(dev_f32(g.ravel()[:count]), dev_f32(u.ravel()[:count]))
        assert np.array_equal(h.view(torch.int16).cpu().numpy().view(np.uint16),
                              oracle.relu2_glu(g.ravel()[:count], u.ravel()[:count]))


# --------------------------------------------------------- fused entries ----

@pytest.mark.parametrize("M,K,N1,N2", [(1, 2560, 6912, 6912), (4, 3200, 8640, 8640),
                                       (16, 2560, 200, 57), (40, 320, 300, 129)])
def test_bitlinear_pair_matches_two_calls_and_oracle(M, K, N1, N2):
    q1, xq, xs, g1 = _product_case(M, K, N1, 60)
    rng = np.random.default_rng(61)
    q2 = rand_codes(rng, N2, K)
    g2 = np.float32(0.0203)
    args = (torch.from_numpy(xq).to(DEV), dev_f32(xs))
    W1, W2 = dev_packed(oracle.pack(q1)), dev_packed(oracle.pack(q2))
    G1, G2 = dev_f32([g1]), dev_f32([g2])
    y1, y2 = bl.bitlinear_pair(*args, W1, G1, W2, G2)
    r1 = bl.bitlinear(*args, W1, G1)
    r2 = bl.bitlinear(*args, W2, G2)
    assert torch.equal(y1.view(torch.int32), r1.view(torch.int32))
    assert torch.equal(y2.view(torch.int32), r2.view(torch.int32))
    assert_y_close(y1.cpu().numpy(), oracle.bitlinear(xq, xs, q1, g1)[0], "pair 1")
    assert_y_close(y2.cpu().numpy(), oracle.bitlinear(xq, xs, q2, g2)[0], "pair 2")


@pytest.mark.parametrize("M,K", [(1, 6912), (4, 6912), (16, 8640), (3, 64), (2, 28672),
                                 (300, 2560)])
def test_relu2_glu_quant_matches_oracle(M, K):
    g, u = wl.ffn_hidden(62, K, M, K)
    hq, hs = bl.relu2_glu_quant(dev_f32(g), dev_f32(u))
    h_ref = oracle.relu2_glu(g, u)
    hq_ref, hs_ref = oracle.act_quant(h_ref)
    assert np.array_equal(hq.cpu().numpy(), hq_ref)
    assert np.array_equal(hs.cpu().numpy(), hs_ref)
    # Same bits as the two unfused calls.
    h = bl.relu2_glu(dev_f32(g), dev_f32(u))
    hq2, hs2 = bl.quantize_acts(h)
    assert torch.equal(hq, hq2) and torch.equal(hs, hs2)


def test_ffn_block_fused_path_equals_unfused():
    """Decode FFN step through the fused entry points gives the same bits as
    the unfused sequence (which the stage-wise test checks against the oracle)."""
    wid = 2
    _, projs, _ = wl.WORKLOADS[wid]
    dev = {name: gpu_weights(wl.weights(wid, i, N, K)) for i, (name, K, N) in enumerate(projs)}
    for M in (1, 4, 16):
        x = dev_bf16(wl.activations(wid, 9, M, 2560))
        xq, xs = bl.quantize_acts(x)
        yg, yu = bl.bitlinear_pair(xq, xs, *dev["gate"], *dev["up"])
        hq, hs = bl.relu2_glu_quant(yg, yu)
        y = bl.bitlinear(hq, hs, *dev["down"])
        rg = bl.bitlinear(xq, xs, *dev["gate"])
        ru = bl.bitlinear(xq, xs, *dev["up"])
        rq, rs = bl.quantize_acts(bl.relu2_glu(rg, ru))
        ry = bl.bitlinear(rq, rs, *dev["down"])
        assert torch.equal(hq, rq) and torch.equal(hs, rs)
        assert torch.equal(y.view(torch.int32), ry.view(torch.int32))


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 16, 40])
@pytest.mark.parametrize("K,N_ff", [(2560, 6912), (3200, 8640), (512, 1024), (1024, 2624)])
def test_ffn_relu2_matches_unfused_sequence(M, K, N_ff):
    """bl_ffn_relu2 (two launches for M in 1, 2, 4, 8; three at 16: gate/up,
    an act quant of h, the down GEMV; four otherwise; N_ff = 2624 leaves a
    16-byte tail on the down projection's rows) gives the bits
    of quantize_acts -> bitlinear(gate, up) -> relu2_glu -> quantize_acts ->
    bitlinear(down); the unfused sequence is checked against the oracle by
    the stage-wise block test."""
    wid = 70
    Wg, Wu = wl.weights(wid, 0, N_ff, K), wl.weights(wid, 1, N_ff, K)
    Wd = wl.weights(wid, 2, K, N_ff)
    (pg, gg), (pu, gu), (pd, gd) = gpu_weights(Wg), gpu_weights(Wu), gpu_weights(Wd)
    x = dev_bf16(wl.activations(wid, M, M, K))
    y = bl.ffn_relu2(x, pg, gg, pu, gu, pd, gd)
    xq, xs = bl.quantize_acts(x)
    h = bl.relu2_glu(bl.bitlinear(xq, xs, pg, gg), bl.bitlinear(xq, xs, pu, gu))
    hq, hs = bl.quantize_acts(h)
    ref = bl.bitlinear(hq, hs, pd, gd)
    assert torch.equal(y.view(torch.int32), ref.view(torch.int32))
    # Second call on the same workspace: no state carried over.
    ws = bl.ffn_relu2_workspace(M, K, N_ff, DEV)
    y2 = bl.ffn_relu2(x, pg, gg, pu, gu, pd, gd, workspace=ws)
    y3 = bl.ffn_relu2(x, pg, gg, pu, gu, pd, gd, workspace=ws)
    assert torch.equal(y2.view(torch.int32), ref.view(torch.int32))
    assert torch.equal(y3.view(torch.int32), ref.view(torch.int32))


def test_ffn_relu2_oracle_end_to_end_small():
    """Fused step against the oracle on its own end-to-end path; the down
    input codes can flip by one at rounding boundaries of y_gate, y_up
    (fp32 within 1e-6), so the check counts flips and bounds y."""
    wid, M, K, N_ff = 71, 4, 512, 1024
    Wg, Wu, Wd = wl.weights(wid, 0, N_ff, K), wl.weights(wid, 1, N_ff, K), wl.weights(wid, 2, K, N_ff)
    xb = wl.activations(wid, 0, M, K)
    (pg, gg), (pu, gu), (pd, gd) = gpu_weights(Wg), gpu_weights(Wu), gpu_weights(Wd)
    y = bl.ffn_relu2(dev_bf16(xb), pg, gg, pu, gu, pd, gd).cpu().numpy()
    _, g_g, q_g = oracle.quantize_weights(Wg)
    _, g_u, q_u = oracle.quantize_weights(Wu)
    _, g_d, q_d = oracle.quantize_weights(Wd)
    xq, xs = oracle.act_quant(xb)
    yg, _ = oracle.bitlinear(xq, xs, q_g, g_g)
    yu, _ = oracle.bitlinear(xq, xs, q_u, g_u)
    hq, hs = oracle.act_quant(oracle.relu2_glu(yg, yu))
    y_ref, _ = oracle.bitlinear(hq, hs, q_d, g_d)
    rel = np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref)
    assert rel < 1e-3, rel


# ---------------------------------------------- sub-layer norm (subln) ----
# h -> RMSNorm(h; g) -> per-token quant before the down projection: the codes
# are those of z = h*g (bit-exact); the scale a / (127 rms) has an fp64 sum
# of squares whose order is the kernel's (within 1e-6 relative).

@pytest.mark.parametrize("M,K", [(1, 6912), (4, 8640), (16, 6912), (3, 64), (300, 2560)])
def test_relu2_glu_subln_quant_matches_oracle(M, K):
    g, u = wl.ffn_hidden(63, K, M, K)
    gain = wl.rms_gain(63, K, K)
    hq, hs = bl.relu2_glu_quant(dev_f32(g), dev_f32(u), subln_gain=dev_bf16(gain))
    hq_ref, hs_ref = oracle.act_quant(oracle.relu2_glu(g, u), gain)
    assert np.array_equal(hq.cpu().numpy(), hq_ref)
    hs = hs.cpu().numpy()
    assert np.all(np.abs(hs - hs_ref) <= RTOL_SCALE_FUSED * hs_ref)
    # The plain glue quant is unchanged by the option.
    hq0, hs0 = bl.relu2_glu_quant(dev_f32(g), dev_f32(u))
    hq0_ref, hs0_ref = oracle.act_quant(oracle.relu2_glu(g, u))
    assert np.array_equal(hq0.cpu().numpy(), hq0_ref) and np.array_equal(hs0.cpu().numpy(), hs0_ref)


@pytest.mark.parametrize("M", [1, 2, 4, 5, 16])
@pytest.mark.parametrize("K,N_ff", [(2560, 6912), (512, 1024)])
def test_ffn_relu2_subln_matches_unfused_sequence(M, K, N_ff):
    """bl_ffn_relu2_subln (two launches for M <= 4, four otherwise) against
    quantize_acts -> bitlinear(gate, up) -> relu2_glu -> quantize_acts(h,
    gain) -> bitlinear(down): the int32 sums agree exactly (same codes), y
    within 1e-6 relative (the scales' fp64 sums differ in order)."""
    wid = 72
    Wg, Wu = wl.weights(wid, 0, N_ff, K), wl.weights(wid, 1, N_ff, K)
    Wd = wl.weights(wid, 2, K, N_ff)
    (pg, gg), (pu, gu), (pd, gd) = gpu_weights(Wg), gpu_weights(Wu), gpu_weights(Wd)
    x = dev_bf16(wl.activations(wid, M, M, K))
    gain = dev_bf16(wl.rms_gain(wid, 0, N_ff))
    y = bl.ffn_relu2(x, pg, gg, pu, gu, pd, gd, subln_gain=gain).cpu().numpy()
    xq, xs = bl.quantize_acts(x)
    h = bl.relu2_glu(bl.bitlinear(xq, xs, pg, gg), bl.bitlinear(xq, xs, pu, gu))
    hq, hs = bl.quantize_acts(h, gain)
    ref, acc = bl.bitlinear(hq, hs, pd, gd, return_acc=True)
    # y / (scale * gamma) recovers the sums: compare them through the scale
    # the reference used, to within the scale tolerance.
    assert_close = np.abs(y.astype(np.float64) - ref.cpu().numpy()) <= \
        RTOL_Y * np.abs(ref.cpu().numpy().astype(np.float64)) + 1e-30
    assert assert_close.all(), float(np.abs(y - ref.cpu().numpy()).max())
    # Without the gain the same call is the plain step (bit-exact as before).
    y0 = bl.ffn_relu2(x, pg, gg, pu, gu, pd, gd)
    hq0, hs0 = bl.quantize_acts(h)
    assert torch.equal(y0.view(torch.int32), bl.bitlinear(hq0, hs0, pd, gd).view(torch.int32))


def test_ffn_subln_down_input_against_oracle():
    """Stage-wise against the oracle: from the GPU's own h, the oracle's
    RMSNorm-fused quantisation gives the codes of the GPU's subln glue quant,
    and the down projection of those codes matches the fused step."""
    wid, M, K, N_ff = 73, 4, 512, 1024
    Wg, Wu, Wd = wl.weights(wid, 0, N_ff, K), wl.weights(wid, 1, N_ff, K), wl.weights(wid, 2, K, N_ff)
    (pg, gg), (pu, gu), (pd, gd) = gpu_weights(Wg), gpu_weights(Wu), gpu_weights(Wd)
    x = dev_bf16(wl.activations(wid, 0, M, K))
    gain_bits = wl.rms_gain(wid, 0, N_ff)
    xq, xs = bl.quantize_acts(x)
    yg, yu = bl.bitlinear(xq, xs, pg, gg), bl.bitlinear(xq, xs, pu, gu)
    hq, hs = bl.relu2_glu_quant(yg, yu, subln_gain=dev_bf16(gain_bits))
    h_bits = bl.relu2_glu(yg, yu).cpu().view(torch.int16).numpy().view(np.uint16)
    hq_ref, hs_ref = oracle.act_quant(h_bits, gain_bits)
    assert np.array_equal(hq.cpu().numpy(), hq_ref)
    assert np.all(np.abs(hs.cpu().numpy() - hs_ref) <= RTOL_SCALE_FUSED * hs_ref)
    _, g_d, q_d = oracle.quantize_weights(Wd)
    y_ref, _ = oracle.bitlinear(hq_ref, hs_ref, q_d, g_d)
    y = bl.ffn_relu2(x, pg, gg, pu, gu, pd, gd, subln_gain=dev_bf16(gain_bits)).cpu().numpy()
    assert np.all(np.abs(y.astype(np.float64) - y_ref) <= RTOL_Y * np.abs(y_ref.astype(np.float64)))


# -------------------------------------------------------------- SwiGLU ----
# h = bf16(fp32(SiLU(g)) * u) with SiLU evaluated in fp64 on both sides. The
# device's fp64 exp and the host's each lie within about an ulp of exp, so
# the two fp32 SiLU values can differ only where the fp64 value sits within
# about 1e-13 of an fp32 rounding boundary; such elements are counted, every
# other h must match bit for bit, and everything downstream is checked
# bit-exactly from the GPU's own h.

def _silu_near_rounding_boundary(g):
    """Gates whose fp64 SiLU lies within 1e-13 relative of an fp32 rounding
    boundary: there the device's and the host's fp64 exp, each within an ulp
    or so of exp, may round SiLU to different fp32 values. Everywhere else
    both sides must give the same bits."""
    g = np.asarray(g, np.float64)
    with np.errstate(over="ignore"):
        s64 = g / (1.0 + np.exp(-g))
    s32 = s64.astype(np.float32)
    nxt = np.where(s64 > s32, np.nextafter(s32, np.float32(np.inf)),
                   np.nextafter(s32, np.float32(-np.inf))).astype(np.float64)
    mid = (s32.astype(np.float64) + nxt) / 2
    return np.abs(s64 - mid) <= 1e-13 * np.abs(s64)


def _h_exact(h_bits, h_ref_bits, g):
    """h bit-exact except at double-rounding exceptions (counted): returns
    (every mismatch is such an exception, mismatches, exceptions)."""
    diff = h_bits != h_ref_bits
    near = _silu_near_rounding_boundary(g)
    return bool(np.all(near[diff])), int(diff.sum()), int(near.sum())


def test_swiglu_parity():
    g, u = wl.ffn_hidden(64, 0, 37, 1024)
    g[0, :10] = [0.0, 1.0, -1.0, 20.0, -20.0, -30.0, -100.0, 100.0, 3.5, -1.2785]
    g[1, :4] = [-700.0, -710.0, -1e30, 1e30]
    u[0, :10] = 1.0
    h = bl.glu(dev_f32(g), dev_f32(u), "swiglu").cpu().view(torch.int16).numpy().view(np.uint16)
    h_ref = oracle.swiglu(g, u)
    ok, differ, near = _h_exact(h, h_ref, g)
    assert ok, f"{differ} of {h.size} h values differ away from rounding boundaries"
    assert differ <= near
    # The two hand values the oracle is pinned to.
    hv = wl.bf16_bits_to_f32(h[0, 1:3])
    assert hv[0] == np.float32(187 / 256) and hv[1] == np.float32(-138 / 512)


@pytest.mark.parametrize("M,K", [(1, 6912), (4, 8640), (16, 2560), (300, 1024)])
def test_swiglu_quant_from_gpu_h(M, K):
    g, u = wl.ffn_hidden(65, K, M, K)
    gain = wl.rms_gain(65, 1, K)
    h_dev = bl.glu(dev_f32(g), dev_f32(u), "swiglu")
    h = h_dev.cpu().view(torch.int16).numpy().view(np.uint16)
    assert _h_exact(h, oracle.swiglu(g, u), g)[0]
    hq, hs = bl.glu_quant(dev_f32(g), dev_f32(u), "swiglu")
    hq_ref, hs_ref = oracle.act_quant(h)
    assert np.array_equal(hq.cpu().numpy(), hq_ref) and np.array_equal(hs.cpu().numpy(), hs_ref)
    hq2, hs2 = bl.quantize_acts(h_dev)
    assert torch.equal(hq, hq2) and torch.equal(hs, hs2)
    hq, hs = bl.glu_quant(dev_f32(g), dev_f32(u), "swiglu", subln_gain=dev_bf16(gain))
    hq_ref, hs_ref = oracle.act_quant(h, gain)
    assert np.array_equal(hq.cpu().numpy(), hq_ref)
    assert np.all(np.abs(hs.cpu().numpy() - hs_ref) <= RTOL_SCALE_FUSED * hs_ref)


@pytest.mark.parametrize("M", [1, 4, 5, 16])
@pytest.mark.parametrize("K,N_ff", [(3200, 8640), (512, 1024)])
def test_ffn_step_swiglu_matches_unfused_sequence(M, K, N_ff):
    """bl_ffn_step with SwiGLU gating (two launches for M in 1, 2, 4, 8, 16, four
    otherwise) against the single calls: bit-exact without the norm, y within
    1e-6 relative with it."""
    wid = 74
    Wg, Wu = wl.weights(wid, 0, N_ff, K), wl.weights(wid, 1, N_ff, K)
    Wd = wl.weights(wid, 2, K, N_ff)
    (pg, gg), (pu, gu), (pd, gd) = gpu_weights(Wg), gpu_weights(Wu), gpu_weights(Wd)
    x = dev_bf16(wl.activations(wid, M, M, K))
    xq, xs = bl.quantize_acts(x)
    yg, yu = bl.bitlinear(xq, xs, pg, gg), bl.bitlinear(xq, xs, pu, gu)
    h = bl.glu(yg, yu, "swiglu")
    hq, hs = bl.quantize_acts(h)
    ref = bl.bitlinear(hq, hs, pd, gd)
    y = bl.ffn_step(x, pg, gg, pu, gu, pd, gd, kind="swiglu")
    assert torch.equal(y.view(torch.int32), ref.view(torch.int32))
    # Stage-wise against the oracle from the GPU's own gate/up outputs.
    h_bits = h.cpu().view(torch.int16).numpy().view(np.uint16)
    assert _h_exact(h_bits, oracle.swiglu(yg.cpu().numpy(), yu.cpu().numpy()),
                    yg.cpu().numpy())[0]
    gain = wl.rms_gain(wid, 0, N_ff)
    hq2, hs2 = bl.quantize_acts(h, dev_bf16(gain))
    ref2 = bl.bitlinear(hq2, hs2, pd, gd).cpu().numpy().astype(np.float64)
    y2 = bl.ffn_step(x, pg, gg, pu, gu, pd, gd, kind="swiglu",
                     subln_gain=dev_bf16(gain)).cpu().numpy()
    assert np.all(np.abs(y2 - ref2) <= RTOL_Y * np.abs(ref2) + 1e-30)
    # The relu2 kind of the general entry is bl_ffn_relu2 bit for bit.
    y3 = bl.ffn_step(x, pg, gg, pu, gu, pd, gd, kind="relu2")
    assert torch.equal(y3.view(torch.int32), bl.ffn_relu2(x, pg, gg, pu, gu, pd, gd).view(torch.int32))


# --------------------------------------------------------- calibration ----

def test_calibration_kernels():
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (1 << 20,), dtype=torch.int32, device=DEV)
    dst = torch.zeros_like(src)
    bl.calib_copy(dst, src)
    assert torch.equal(dst, src)
    tail = torch.zeros(1000 + 4, dtype=torch.int32, device=DEV)  # 16-byte multiple
    bl.calib_copy(tail, src[:1004].clone())
    assert torch.equal(tail, src[:1004])
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    bl.calib_read(src, sink)
    ms = bl.calib_mfma_sink(DEV)
    ops = bl.calib_mfma_i8(3, ms)
    first = ms.clone()
    assert ops == 3 * 8 * 2 * 32 ** 3 * 4 * (ms.numel() // 256)
    bl.calib_mfma_i8(3, ms)
    torch.cuda.synchronize()
    assert torch.equal(first, ms) and int(first.abs().max()) > 0


# ------------------------------------------------- other weight formats ----
# 1-bit {-1, +1} weights and five ternary weights per byte: packers bit-exact
# against the oracle's packing of the oracle's codes, decode products exact in
# int32 and within 1e-6 in fp32, and (base 3) bit-identical to the 2-bit path
# on the same codes.

FORMAT_CASES = [(1, 64, 16), (3, 192, 70), (1, 2560, 300), (16, 6912, 257), (5, 8640, 40),
                (2, 3200, 33), (1, 28672, 48), (4, 8192, 100)]


def _latent(rng, N, K):
    W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    W[0, :8] = [0.0, -0.0, 1e-30, -1e-30, 0.0, -0.0, 0.0, -0.0]   # signs of zeros
    return W


@pytest.mark.parametrize("M,K,N", FORMAT_CASES)
def test_binary_weights_parity(M, K, N):
    rng = np.random.default_rng(M * 1000 + K + N)
    W = _latent(rng, N, K)
    bits_ref, g_ref, q = oracle.quantize_weights_binary(W)
    bits, g = bl.quantize_weights_binary(dev_f32(W))
    assert g.item() == float(g_ref)
    assert np.array_equal(bits.cpu().numpy().view(np.uint32), bits_ref)
    xq, xs = oracle.act_quant(wl.activations(61, 0, M, K))
    y, acc = bl.bitlinear_binary(torch.from_numpy(xq).to(DEV), dev_f32(xs), bits, g,
                                 return_acc=True)
    y_ref, acc_ref = oracle.bitlinear(xq, xs, q, g_ref)
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert_y_close(y.cpu().numpy(), y_ref, "binary")


@pytest.mark.parametrize("M,K,N", FORMAT_CASES)
def test_base3_weights_parity(M, K, N):
    rng = np.random.default_rng(M * 2000 + K + N)
    q = rand_codes(rng, N, K)
    q[0] = 0
    q[-1] = 1
    pk = dev_packed(oracle.pack(q))
    w3 = bl.pack_base3(pk, K)
    assert np.array_equal(w3.cpu().numpy(), oracle.pack_base3(q))
    xq, xs = oracle.act_quant(wl.activations(62, 0, M, K))
    xq_d, xs_d, g = torch.from_numpy(xq).to(DEV), dev_f32(xs), dev_f32([0.0159])
    y, acc = bl.bitlinear_base3(xq_d, xs_d, w3, g, return_acc=True)
    y_ref, acc_ref = oracle.bitlinear(xq, xs, q, np.float32(0.0159))
    assert np.array_equal(acc.cpu().numpy(), acc_ref)
    assert_y_close(y.cpu().numpy(), y_ref, "base3")
    y2, acc2 = bl.bitlinear(xq_d, xs_d, pk, g, return_acc=True, path=1)
    assert torch.equal(acc, acc2) and torch.equal(y.view(torch.int32), y2.view(torch.int32))


# 1-bit rows at one token (the streaming kernel): rows of one piece or less,
# whole pieces, partial last pieces, rows padded to 16 bytes, the longest row.
BINARY_ONE_TOKEN_CASES = [(64, 7), (128, 1), (320, 200), (4160, 33), (8192, 257), (8256, 9),
                          (16384, 3), (28672, 65), (65536, 5)]


@pytest.mark.parametrize("K,N", BINARY_ONE_TOKEN_CASES)
def test_binary_one_token_parity(K, N):
    """bl_bitlinear_binary at one token against the oracle (int32 sums exact, y
    within 1e-6) on random +-1 codes with an all-(+1) and an all-(-1) row, for
    the extreme +127 and -128 tokens, a full-range token and a quantised one."""
    rng = np.random.default_rng(K * 11 + N)
    q = np.where(rng.random((N, K)) < 0.5, -1, 1).astype(np.int8)
    q[0] = 1
    q[-1] = -1
    packed = oracle.pack_binary(q)
    bits = torch.from_numpy(packed.view(np.int32)).to(DEV)
    xq_h, xs_h = oracle.act_quant(wl.activations(64, 1, 1, K))
    tokens = [np.full((1, K), 127, np.int8), np.full((1, K), -128, np.int8),
              rng.integers(-128, 128, (1, K)).astype(np.int8), xq_h]
    g = dev_f32([0.0211])
    for t in tokens:
        y, acc = bl.bitlinear_binary(torch.from_numpy(t).to(DEV), dev_f32(xs_h), bits, g,
                                     return_acc=True)
        y_ref, acc_ref = oracle.bitlinear(t, xs_h, q, np.float32(0.0211))
        assert np.array_equal(acc.cpu().numpy(), acc_ref)
        assert_y_close(y.cpu().numpy(), y_ref, f"binary one token K={K}")


# Base-3 rows at one token: short rows, K not a multiple of 5 or 16 bytes of
# row, 8192 and 28672 columns, and long rows.
BASE3_ONE_TOKEN_CASES = [(64, 7), (320, 200), (4160, 33), (8192, 257), (8256, 9), (12800, 3),
                         (28672, 65), (61440, 17), (61504, 5)]


@pytest.mark.parametrize("K,N", BASE3_ONE_TOKEN_CASES)
def test_base3_one_token_parity(K, N):
    """bl_bitlinear_base3 at one token against the oracle (int32 sums exact, y
    within 1e-6) and against the 2-bit path's bits, on random codes with an
    all-zero, an all-(+1) and an all-(-1) row, for the extreme +127 token, a
    full-range token (-128 included) and a quantised one."""
    rng = np.random.default_rng(K * 7 + N)
    q = rand_codes(rng, N, K)
    q[0] = 0
    q[min(1, N - 1)] = 1
    q[-1] = -1
    pk = dev_packed(oracle.pack(q))
    w3 = bl.pack_base3(pk, K)
    assert np.array_equal(w3.cpu().numpy(), oracle.pack_base3(q))
    xq_h, xs_h = oracle.act_quant(wl.activations(63, 1, 1, K))
    tokens = [np.full((1, K), 127, np.int8), rng.integers(-128, 128, (1, K)).astype(np.int8), xq_h]
    g = dev_f32([0.0137])
    for t in tokens:
        xd, xsd = torch.from_numpy(t).to(DEV), dev_f32(xs_h)
        y, acc = bl.bitlinear_base3(xd, xsd, w3, g, return_acc=True)
        y_ref, acc_ref = oracle.bitlinear(t, xs_h, q, np.float32(0.0137))
        assert np.array_equal(acc.cpu().numpy(), acc_ref)
        assert_y_close(y.cpu().numpy(), y_ref, f"base3 one token K={K}")
        y2, acc2 = bl.bitlinear(xd, xsd, pk, g, return_acc=True)
        assert torch.equal(acc, acc2) and torch.equal(y.view(torch.int32), y2.view(torch.int32))


@pytest.mark.parametrize("idx", [0, 1])
def test_other_formats_70b_full_size(idx):
    """70B-class matrices at full size, M = 1: base 3 repacked from the
    workload's 2-bit weights gives the 2-bit path's bits; binary weights of the
    same latent matrix against the oracle on sampled rows."""
    q_ref, g_ref, pk, g = workload_weights(5, idx)
    _, K, N = wl.WORKLOADS[5][1][idx]
    x = wl.activations(5, idx, 1, K)
    xq, xs = bl.quantize_acts(dev_bf16(x))
    w3 = bl.pack_base3(pk, K)
    rows = np.sort(np.random.default_rng(idx).choice(N, 64, replace=False))
    assert np.array_equal(w3[torch.from_numpy(rows).to(DEV)].cpu().numpy(),
                          oracle.pack_base3(q_ref[rows]))
    y3, a3 = bl.bitlinear_base3(xq, xs, w3, g, return_acc=True)
    y2, a2 = bl.bitlinear(xq, xs, pk, g, return_acc=True)
    assert torch.equal(a3, a2) and torch.equal(y3.view(torch.int32), y2.view(torch.int32))
    W = wl.weights(5, idx, N, K)
    bits, gb = bl.quantize_weights_binary(dev_f32(W))
    assert gb.item() == float(g_ref)
    qb = oracle.binarize(W[rows])
    del W
    assert np.array_equal(bits[torch.from_numpy(rows).to(DEV)].cpu().numpy().view(np.uint32),
                          oracle.pack_binary(qb))
    yb, ab = bl.bitlinear_binary(xq, xs, bits, gb, return_acc=True)
    yr, ar = oracle.bitlinear(xq.cpu().numpy(), xs.cpu().numpy(), qb, g_ref)
    idx_t = torch.from_numpy(rows).to(DEV)
    assert np.array_equal(ab[:, idx_t].cpu().numpy(), ar)
    assert_y_close(yb[:, idx_t].cpu().numpy(), yr, "binary 70B")


def test_other_formats_reject_prefill_sizes():
    q = np.zeros((16, 64), np.int8)
    pk = dev_packed(oracle.pack(q))
    w3 = bl.pack_base3(pk, 64)
    xq = torch.zeros((17, 64), dtype=torch.int8, device=DEV)
    xs = torch.ones(17, device=DEV)
    with pytest.raises(bl.BitLinearError):
        bl.bitlinear_base3(xq, xs, w3, dev_f32([1.0]))


# ------------------------------------------- straight-through backward ----
# dx = gamma * dy . q: transposed codes bit-exact; dx within the fp32
# summation bound of the exact value (the products bf16 x {-1, 0, +1} are
# exact; N fp32 additions each within 2^-24 of the running sum, then one
# rounding of the product with gamma).

def _dx_bound(dy_bits, q, g):
    absdy = np.abs(wl.bf16_bits_to_f32(dy_bits).astype(np.float64))
    mag = float(g) * (absdy @ np.abs(q.astype(np.float64)))
    N = q.shape[0]
    return (N * 2.0 ** -24 + 2.0 ** -23) * mag + 1e-30


STE_CASES = [(1, 8, 64), (3, 40, 128), (130, 264, 192), (64, 2560, 640), (17, 6912, 256)]


@pytest.mark.parametrize("M,N,K", STE_CASES)
def test_ste_backward_dx_parity(M, N, K):
    rng = np.random.default_rng(M + 7 * N + K)
    q = rand_codes(rng, N, K)
    q[:, 0] = 1
    q[:, -1] = 0
    g = np.float32(0.0173)
    qT_ref = oracle.pack_ste_t(q)
    qT = bl.pack_ste_t(dev_packed(oracle.pack(q)), K)
    assert np.array_equal(qT.cpu().numpy(), qT_ref)
    dy = wl.f32_to_bf16_bits((rng.standard_normal((M, N)) * 0.01).astype(np.float32))
    dx = bl.ste_backward_dx(dev_bf16(dy), qT, dev_f32([g]), N).cpu().numpy()
    ref = oracle.ste_dx(dy, q, g)
    err = np.abs(dx.astype(np.float64) - ref.astype(np.float64))
    assert (err <= _dx_bound(dy, q, g)).all(), float(err.max())


def test_ste_backward_dx_large_tiles_ragged():
    """128 x 512 output tiles (2000 x 4800 is 160 of them, 128-wide reduction
    stages), ragged in tokens, input features and the reduction: N = 264
    leaves 8 valid n in the third stage, and the second 16 bytes of that
    stage's codes lie past the 80-byte rows; oracle on sampled token rows,
    all K."""
    M, N, K = 2000, 264, 4800
    rng = np.random.default_rng(97)
    q = rand_codes(rng, N, K)
    g = np.float32(0.0211)
    qT = bl.pack_ste_t(dev_packed(oracle.pack(q)), K)
    dy = wl.f32_to_bf16_bits((rng.standard_normal((M, N)) * 0.01).astype(np.float32))
    dx = bl.ste_backward_dx(dev_bf16(dy), qT, dev_f32([g]), N)
    edges = [m for t in range(0, M, 128) for m in (t, min(t + 127, M - 1))]
    rows = np.unique(np.concatenate([edges[:4], edges[-4:], rng.choice(M, 8, replace=False)]))
    ref = oracle.ste_dx(dy[rows], q, g)
    got = dx[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    assert (err <= _dx_bound(dy[rows], q, g)).all(), float(err.max())


# dW: tokens ragged against the 64-token padding, features ragged against the
# 128 x 256 tiles and the 64-wide stages. The last two have more tiles than
# CUs with a last round at most half full (612 and 273 tiles), so their last
# row tiles go through the second launch of 64 x 64 tiles (760 and 168 rows).
STE_DW_CASES = [(1, 8, 64), (3, 40, 128), (70, 136, 320), (200, 264, 576), (64, 128, 256),
                (130, 520, 704), (257, 1000, 1344), (70, 4344, 4608), (33, 2600, 3328)]


def _dw_bound(dy_bits, xq, xs):
    """(2^-16 + 2^-24 + 2 Mp 2^-24) * sum_m |dy x_q x_scale| per element: the
    split of dy * x_scale into two bf16 parts, its fp32 rounding, and fp32
    accumulation of 2 Mp exact products."""
    M = dy_bits.shape[0]
    Mp = (M + 63) // 64 * 64
    a = np.abs(wl.bf16_bits_to_f32(dy_bits).astype(np.float64) * xs.astype(np.float64)[:, None])
    mag = a.T @ np.abs(xq.astype(np.float64))
    return (2.0 ** -16 + 2.0 ** -24 + 2 * Mp * 2.0 ** -24) * mag + 1e-30


def _dw_case(M, N, K, seed):
    rng = np.random.default_rng(seed)
    dy = wl.f32_to_bf16_bits((rng.standard_normal((M, N)) * 0.01).astype(np.float32))
    x = wl.activations(seed % 1000, 1, M, K)
    xq, xs = oracle.act_quant(x)
    return dy, xq, xs


@pytest.mark.parametrize("M,N,K", STE_DW_CASES)
def test_ste_backward_dw_parity(M, N, K):
    """dW against the oracle's exact fp64 sum, within the derived fp32 bound."""
    dy, xq, xs = _dw_case(M, N, K, 90 + M)
    ref = oracle.ste_dw(dy, xq, xs).astype(np.float64)
    dW = bl.ste_backward_dw(dev_bf16(dy), torch.from_numpy(xq).to(DEV), dev_f32(xs))
    err = np.abs(dW.cpu().numpy().astype(np.float64) - ref)
    assert (err <= _dw_bound(dy, xq, xs)).all(), float((err / _dw_bound(dy, xq, xs)).max())


def test_ste_backward_dw_exact_cases():
    """Where every value is exact (power-of-two scales, small sums) dW is the
    oracle's bit for bit; a one-hot dy gives one token's dequantised row
    within the split's 2^-16 (the two bf16 parts keep 16 of the scale's 24
    significant bits) and exact zeros elsewhere."""
    M, N, K = 96, 64, 128
    rng = np.random.default_rng(93)
    dy = wl.f32_to_bf16_bits(rng.integers(-4, 5, (M, N)).astype(np.float32))
    xq = rng.integers(-128, 128, (M, K)).astype(np.int8)
    xs = (2.0 ** -rng.integers(3, 9, M)).astype(np.float32)
    dW = bl.ste_backward_dw(dev_bf16(dy), torch.from_numpy(xq).to(DEV), dev_f32(xs))
    assert np.array_equal(dW.cpu().numpy(), oracle.ste_dw(dy, xq, xs))
    d1 = np.zeros((M, N), np.float32)
    d1[37, 11] = 1.0
    xs2 = (rng.random(M) * 0.05 + 0.001).astype(np.float32)
    dW1 = bl.ste_backward_dw(dev_bf16(wl.f32_to_bf16_bits(d1)), torch.from_numpy(xq).to(DEV),
                             dev_f32(xs2)).cpu().numpy()
    ref1 = oracle.ste_dw(wl.f32_to_bf16_bits(d1), xq, xs2).astype(np.float64)
    assert (np.abs(dW1[11] - ref1[11]) <= 2.0 ** -16 * np.abs(ref1[11])).all()
    assert (np.delete(dW1, 11, axis=0) == 0).all()


@pytest.mark.parametrize("idx", [0, 1])
def test_ste_backward_dw_full_size(idx):
    """The 4096-token shapes: every element against an fp64 product of the
    same operands (exact products; fp64 sums), within the derived bound; 16
    rows through the oracle itself; three calls give the same bits."""
    _, projs, Ms = wl.WORKLOADS[3]
    name, K, N = projs[idx]
    M = Ms[0]
    dy, xq, xs = _dw_case(M, N, K, 95 + idx)
    args = (dev_bf16(dy), torch.from_numpy(xq).to(DEV), dev_f32(xs))
    ws = bl.ste_dw_workspace(M, N, K, DEV)
    dW = bl.ste_backward_dw(*args, workspace=ws)
    got = dW.cpu().numpy().astype(np.float64)
    a = wl.bf16_bits_to_f32(dy).astype(np.float64) * xs.astype(np.float64)[:, None]
    ref = a.T @ xq.astype(np.float64)
    bound = _dw_bound(dy, xq, xs)
    assert (np.abs(got - ref) <= bound).all()
    ns = np.sort(np.random.default_rng(96).choice(N, 16, replace=False))
    ref_o = oracle.ste_dw(np.ascontiguousarray(dy[:, ns]), xq, xs).astype(np.float64)
    assert (np.abs(got[ns] - ref_o) <= bound[ns]).all()
    for _ in range(2):
        again = bl.ste_backward_dw(*args, workspace=ws)
        assert torch.equal(again.view(torch.int32), dW.view(torch.int32))



def test_ste_backward_dw_split_tail():
    """512 tokens, 2600 x 3328: 273 tiles of 128 x 256, so the last two row
    tiles (rows 2432..2599) split their stages over two workgroups and a
    third launch adds the partial tiles. Every element against an fp64
    product of the same operands within the derived bound; rows on both
    sides of the tail boundary through the oracle itself; three calls give
    the same bits."""
    M, N, K = 512, 2600, 3328
    dy, xq, xs = _dw_case(M, N, K, 97)
    args = (dev_bf16(dy), torch.from_numpy(xq).to(DEV), dev_f32(xs))
    ws = bl.ste_dw_workspace(M, N, K, DEV)
    assert ws.numel() == 4 * N * M + 2 * K * M + 2 * 256 * K * 4   # A, B, two partial tiles
    dW = bl.ste_backward_dw(*args, workspace=ws)
    got = dW.cpu().numpy().astype(np.float64)
    a = wl.bf16_bits_to_f32(dy).astype(np.float64) * xs.astype(np.float64)[:, None]
    ref = a.T @ xq.astype(np.float64)
    bound = _dw_bound(dy, xq, xs)
    assert (np.abs(got - ref) <= bound).all(), float((np.abs(got - ref) / bound).max())
    ns = np.array([0, 1000, 2430, 2431, 2432, 2433, 2500, 2598, 2599])
    ref_o = oracle.ste_dw(np.ascontiguousarray(dy[:, ns]), xq, xs).astype(np.float64)
    assert (np.abs(got[ns] - ref_o) <= bound[ns]).all()
    for _ in range(2):
        again = bl.ste_backward_dw(*args, workspace=ws)
        assert torch.equal(again.view(torch.int32), dW.view(torch.int32))

def test_ste_pack_odd_n():
    rng = np.random.default_rng(91)
    q = rand_codes(rng, 37, 64)
    qT = bl.pack_ste_t(dev_packed(oracle.pack(q)), 64)
    assert np.array_equal(qT.cpu().numpy(), oracle.pack_ste_t(q))


@pytest.mark.parametrize("idx", [0, 1])
def test_ste_backward_full_size(idx):
    """The 4096-token workload's projections: dx for a 4096 x N gradient,
    oracle on sampled token rows (all K), transposed codes compared in full."""
    q_ref, g_ref, pk, g = workload_weights(3, idx)
    N, K = q_ref.shape
    qT = bl.pack_ste_t(pk, K)
    assert np.array_equal(qT.cpu().numpy(), oracle.pack_ste_t(q_ref))
    rng = np.random.default_rng(95 + idx)
    M = 4096
    dy = wl.f32_to_bf16_bits((rng.standard_normal((M, N)) * 0.01).astype(np.float32))
    dx = bl.ste_backward_dx(dev_bf16(dy), qT, g, N)
    rows = np.unique(np.concatenate([[0, 127, 128, M - 1], rng.choice(M, 6, replace=False)]))
    ref = oracle.ste_dx(dy[rows], q_ref, g_ref)
    got = dx[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    assert (err <= _dx_bound(dy[rows], q_ref, g_ref)).all(), float(err.max())


# ------------------------------------------------------------ HIP graphs ----
# The benchmark replays captured graphs. Every path it captures is replayed
# several times, with eager work and synchronisations in between, and each
# replay must give the eager result bit for bit (split K zeroes its output
# with a kernel, not a memset node).

def test_graph_replays_match_eager():
    rng = np.random.default_rng(97)
    cases = []
    for (M, K, N) in [(1, 2560, 6912), (16, 6912, 2560), (64, 8192, 700), (300, 2560, 1000)]:
        q = rand_codes(rng, N, K)
        xq, xs = oracle.act_quant(wl.activations(97, 0, M, K))
        cases.append((torch.from_numpy(xq).to(DEV), dev_f32(xs), dev_packed(oracle.pack(q)),
                      dev_f32([0.0159]), torch.empty((M, N), dtype=torch.float32, device=DEV)))
    W = {n: gpu_weights(wl.weights(2, i, N, K)) for i, (n, K, N) in enumerate(wl.WORKLOADS[2][1])}
    ffn_io = []
    for M in (1, 4, 16):
        x = dev_bf16(wl.activations(2, 9, M, 2560))
        ffn_io.append((x, bl.ffn_relu2_workspace(M, 2560, 6912, DEV),
                       torch.empty((M, 2560), dtype=torch.float32, device=DEV)))

    def run():
        for xq, xs, pk, g, y in cases:
            bl.bitlinear(xq, xs, pk, g, out=y)
        for x, ws, y in ffn_io:
            bl.ffn_relu2(x, *W["gate"], *W["up"], *W["down"], workspace=ws, out=y)

    run()
    torch.cuda.synchronize()
    ref = [c[-1].clone() for c in cases] + [io[-1].clone() for io in ffn_io]
    outs = [c[-1] for c in cases] + [io[-1] for io in ffn_io]
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        run()
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        gr.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"replay {rep}"
        run()                       # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.gpu
def test_calls_on_two_streams_do_not_interfere():
    """The same work issued on two streams at once (default priority, no
    synchronisation between them, three rounds) gives the bits of the calls
    run one after another: the library keeps no state that two calls share.
    Covers the GEMV, the GEMM's K-group, split-K and large-tile variants, and
    the FFN step at 1 and 16 tokens (each stream with its own workspace)."""
    gen = torch.Generator(device=DEV)
    gen.manual_seed(77)
    shapes = [(1, 2560, 6912), (16, 6912, 2560), (512, 3200, 3200), (64, 8192, 700),
              (2048, 2560, 2560)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    jobs = []  # per stream: (inputs, reference) pairs
    for _ in streams:
        mine = []
        for M, K, N in shapes:
            pk, g = bl.quantize_weights(torch.randn(N, K, generator=gen, device=DEV) * 0.02)
            xq, xs = bl.quantize_acts(torch.randn(M, K, generator=gen, device=DEV).to(torch.bfloat16))
            mine.append(("bitlinear", (xq, xs, pk, g), bl.bitlinear(xq, xs, pk, g)))
        for M in (1, 16):
            K, N_ff = 2560, 6912
            W = [bl.quantize_weights(torch.randn(n, k, generator=gen, device=DEV) * 0.02)
                 for n, k in ((N_ff, K), (N_ff, K), (K, N_ff))]
            x = torch.randn(M, K, generator=gen, device=DEV).to(torch.bfloat16)
            ws = bl.ffn_relu2_workspace(M, K, N_ff, DEV)
            args = (x, *W[0], *W[1], *W[2])
            mine.append(("ffn", (args, ws), bl.ffn_relu2(*args, workspace=ws)))
        jobs.append(mine)
    torch.cuda.synchronize()
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = [[None] * len(j) for j in jobs]
    for _ in range(3):
        for i in range(len(jobs[0])):
            for si, s in enumerate(streams):
                kind, a, _ref = jobs[si][i]
                with torch.cuda.stream(s):
                    if kind == "bitlinear":
                        outs[si][i] = bl.bitlinear(*a)
                    else:
                        args, ws = a
                        outs[si][i] = bl.ffn_relu2(*args, workspace=ws)
    torch.cuda.synchronize()
    for si in range(len(streams)):
        for i, (kind, _a, ref) in enumerate(jobs[si]):
            assert torch.equal(outs[si][i].view(torch.int32), ref.view(torch.int32)), (si, i, kind)


@pytest.mark.gpu
def test_pending_hip_error_is_not_reported_as_the_calls_own():
    """A non-sticky HIP error left by an unrelated call (hipSetDevice on a
    device that does not exist, which changes nothing) does not turn the next
    library call into BL_ERR_HIP: the call clears it before enqueuing, runs,
    and leaves no pending error behind."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    x = torch.randn(3, 2560, device=DEV).to(torch.bfloat16)
    ref_q, ref_s = bl.quantize_acts(x)
    torch.cuda.synchronize()
    # No torch kernel may run from here to the library call: torch would
    # report the pending error itself.
    assert hip.hipSetDevice(ctypes.c_int(9999)) != 0    # leaves a pending error
    xq, xs = bl.quantize_acts(x)                         # raises on BL_ERR_HIP
    assert hip.hipGetLastError() == 0
    torch.cuda.synchronize()
    assert torch.equal(xq, ref_q) and torch.equal(xs.view(torch.int32), ref_s.view(torch.int32))
