"""GPU parity of the building blocks, through the C-ABI test hooks that run
the production device functions: packed-row unpacking and int32 block dots
(bit-exact), the exponential, Q8_0 and router logits (bit-exact binary32)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import q, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "no GPU visible"
    return t


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("cols", [32, 96, 2048, 6144])
def test_unpack_bitexact(torch, bits, cols):
    say(f"unpack bits={bits} cols={cols}")
    lo, hi = {8: (-128, 127), 4: (-8, 7), 2: (-2, 1)}[bits]
    rng = np.random.default_rng(bits * 1000 + cols)
    rows = 37
    codes = rng.integers(lo, hi + 1, size=(rows, cols)).astype(np.int8)
    codes[0, :] = np.resize(np.arange(lo, hi + 1), cols)
    packed = synth.pack_codes(codes, bits)
    src = torch.from_numpy(packed).cuda()
    out = torch.empty((rows, cols), dtype=torch.int8, device="cuda")
    q().coli_moe_debug_unpack(bits, rows, cols, src, out)
    got = out.cpu().numpy()
    want = np.stack([oracle.unpack(packed[r], cols, bits) for r in range(rows)])
    assert np.array_equal(got, want)
    assert np.array_equal(got, codes)


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_block_dots_bitexact(torch, bits):
    say(f"block dots bits={bits}")
    lo, hi = {8: (-128, 127), 4: (-8, 7), 2: (-2, 1)}[bits]
    rng = np.random.default_rng(50 + bits)
    rows, cols = 64, 6144
    codes = rng.integers(lo, hi + 1, size=(rows, cols)).astype(np.int8)
    codes[1, :] = lo
    qv = rng.integers(-127, 128, size=cols).astype(np.int8)
    qv[:32] = -127
    packed = synth.pack_codes(codes, bits)
    out = torch.empty((rows, cols // 32), dtype=torch.int32, device="cuda")
    q().coli_moe_debug_block_dots(bits, rows, cols, torch.from_numpy(packed).cuda(),
                                  torch.from_numpy(qv).cuda(), out)
    got = out.cpu().numpy()
    for r in range(rows):
        cr = oracle.unpack(packed[r], cols, bits)
        want = [oracle.block_isum(cr[32 * b:32 * b + 32], qv[32 * b:32 * b + 32]) for b in range(cols // 32)]
        assert got[r].tolist() == want


def test_expf_bitexact_on_sweep(torch):
    say("expf sweep")
    bits = np.arange(-2 ** 31, 2 ** 31, 211, dtype=np.int64).astype(np.int32)
    x = bits.view(np.float32)
    x = np.concatenate([x[np.isfinite(x) & (np.abs(x) < 110)],
                        np.float32([0.0, -0.0, np.inf, -np.inf, 88.72283172607422, 88.72283935546875,
                                    -103.97207641601562, -103.97208404541016, -87.5, -100.0])])
    xd = torch.from_numpy(x).cuda()
    yd = torch.empty_like(xd)
    q().coli_moe_debug_expf(xd, yd)
    got = yd.cpu().numpy()
    want = oracle.expf(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_q8_0_bitexact(torch):
    say("q8_0")
    rng = np.random.default_rng(9)
    v = (rng.normal(size=(64, 2048)) * rng.lognormal(size=(64, 1)) * 3).astype(np.float32)
    v[0, :32] = 0.0                     # zero block
    v[1, :32] = 0.5                     # constant block
    v[2, :32] = np.float32(1e-40)       # denormal block
    v[3, 5] = 127.0
    v[3, 6:10] = [2.5, -2.5, 0.5, -0.5]  # half-way codes (amax 127 -> d = 1)
    v[3, :5] = 0.0
    v[3, 10:32] = 0.0
    vd = torch.from_numpy(v).cuda()
    qd = torch.empty((64, 2048), dtype=torch.int8, device="cuda")
    dd = torch.empty((64, 64), dtype=torch.float32, device="cuda")
    q().coli_moe_debug_q8_0(vd, qd, dd)
    wq, wd = oracle.q8_0(v)
    assert np.array_equal(qd.cpu().numpy(), wq)
    assert np.array_equal(dd.cpu().numpy().view(np.uint32), wd.view(np.uint32))


@pytest.mark.parametrize("spec", [synth.TINY, synth.GLM], ids=["tiny", "glm"])
def test_router_logits_bitexact(torch, spec):
    say(f"logits H={spec.hidden} E={spec.n_experts}")
    d = synth.layer_inputs(3, 0, spec, 4)
    x, W = d["x"], d["router_w"]
    logits = torch.empty((4, spec.n_experts), dtype=torch.float32, device="cuda")
    q().coli_moe_debug_logits(q().make_dims(spec), torch.from_numpy(x).cuda(), torch.from_numpy(W).cuda(), logits)
    got = logits.cpu().numpy()
    es = range(spec.n_experts) if spec.n_experts <= 16 else range(0, spec.n_experts, 7)
    for t in range(4):
        for e in es:
            assert got[t, e].view(np.uint32) == oracle.router_logit(x[t], W[e]).view(np.uint32), (t, e)


def test_mfma_i8_lane_layout(torch):
    """The lane layout the prefill kernels assume for v_mfma_i32_32x32x32_i8
    reproduces a host int matmul of the matrices it implies."""
    say("mfma i8 32x32x32 lane layout")
    rng = np.random.default_rng(11)
    a_raw = rng.integers(-128, 128, size=(64, 16), dtype=np.int8)
    b_raw = rng.integers(-128, 128, size=(64, 16), dtype=np.int8)
    c = torch.zeros((64, 16), dtype=torch.int32, device="cuda")
    q().coli_moe_debug_mfma_i8(torch.from_numpy(a_raw).cuda(), torch.from_numpy(b_raw).cuda(), c)
    got = c.cpu().numpy()
    A = np.zeros((32, 32), np.int64)
    B = np.zeros((32, 32), np.int64)
    for lane in range(64):
        for j in range(16):
            A[lane % 32, 16 * (lane // 32) + j] = a_raw[lane, j]
            B[16 * (lane // 32) + j, lane % 32] = b_raw[lane, j]
    C = A @ B
    want = np.zeros((64, 16), np.int64)
    for lane in range(64):
        for r in range(16):
            want[lane, r] = C[8 * (r // 4) + 4 * (lane // 32) + r % 4, lane % 32]
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} lane registers differ, first (lane, register) {bad[:4].tolist()}"


def test_mfma_i8_16x16_lane_layout(torch):
    """The lane layout the prefill kernels' tiles of at most 16 pairs assume
    for v_mfma_i32_16x16x32_i8 reproduces a host int matmul of the matrices
    it implies."""
    say("mfma i8 16x16x32 lane layout")
    rng = np.random.default_rng(13)
    a_raw = rng.integers(-128, 128, size=(64, 8), dtype=np.int8)
    b_raw = rng.integers(-128, 128, size=(64, 8), dtype=np.int8)
    c = torch.zeros((64, 4), dtype=torch.int32, device="cuda")
    q().coli_moe_debug_mfma_i8_16(torch.from_numpy(a_raw).cuda(), torch.from_numpy(b_raw).cuda(), c)
    got = c.cpu().numpy()
    A = np.zeros((16, 32), np.int64)
    B = np.zeros((32, 16), np.int64)
    for lane in range(64):
        for j in range(8):
            A[lane % 16, 8 * (lane // 16) + j] = a_raw[lane, j]
            B[8 * (lane // 16) + j, lane % 16] = b_raw[lane, j]
    C = A @ B
    want = np.zeros((64, 4), np.int64)
    for lane in range(64):
        for r in range(4):
            want[lane, r] = C[4 * (lane // 16) + r, lane % 16]
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} lane registers differ, first (lane, register) {bad[:4].tolist()}"


def _e4m3(byte: int, bias: int = 7) -> float:
    """OCP FP8 E4M3 (bias 7; S.1111.111 is NaN), or with bias 8 the older
    variant, for the diagnostics."""
    s = -1.0 if byte & 0x80 else 1.0
    e, m = (byte >> 3) & 15, byte & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** (1 - bias)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - bias)


def _e2m1(code: int) -> float:
    s = -1.0 if code & 8 else 1.0
    e, m = (code >> 1) & 3, code & 1
    return s * (m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))


def _k_fp8(half: int, j: int) -> int:
    """K of byte j of an FP8 operand in lane half `half`: bytes 0-15 belong
    to the first 32-deep scale block, bytes 16-31 to the second, and the two
    lane halves hold the two 16-element halves of each block."""
    return 32 * (j // 16) + 16 * half + j % 16


def _mfma_f8f6f4_model(fmt_a, a_raw, b_raw, sa, sb, bias=7):
    """C of one scaled 32x32x64 MFMA under the assumed lane layout (float64).
    FP4 A: lane half h holds scale block h, its 32 elements as the nibbles of
    its first 16 bytes (element j: byte j / 2, even j in the low nibble).
    The scale of row (column) i and block kb comes from lane 32 kb + i."""
    A = np.zeros((32, 64))
    B = np.zeros((64, 32))
    SA = np.zeros((32, 2))
    SB = np.zeros((32, 2))
    for lane in range(64):
        i, half = lane % 32, lane // 32
        for j in range(32):
            if fmt_a == 4:
                byte = int(a_raw[lane, j // 2])
                A[i, 32 * half + j] = _e2m1(byte & 15 if j % 2 == 0 else byte >> 4)
            else:
                A[i, _k_fp8(half, j)] = _e4m3(int(a_raw[lane, j]), bias)
            B[_k_fp8(half, j), i] = _e4m3(int(b_raw[lane, j]), bias)
        SA[i, half] = 2.0 ** (int(sa[lane]) - 127)
        SB[i, half] = 2.0 ** (int(sb[lane]) - 127)
    C = np.zeros((32, 32))
    for kb in range(2):
        C += (SA[:, kb:kb + 1] * SB[:, kb][None, :]) * (A[:, 32 * kb:32 * kb + 32] @ B[32 * kb:32 * kb + 32, :])
    want = np.zeros((64, 16))
    for lane in range(64):
        for r in range(16):
            want[lane, r] = C[8 * (r // 4) + 4 * (lane // 32) + r % 4, lane % 32]
    return want


@pytest.mark.parametrize("fmt_a", [0, 4])
def test_mfma_f8f6f4_lane_layout_and_scales(torch, fmt_a):
    """The lane layout and E8M0 scaling the MXFP4 prefill kernels assume for
    v_mfma_scale_f32_32x32x64_f8f6f4 (A FP8 E4M3 or FP4 E2M1, B FP8 E4M3)
    reproduce a float64 host model exactly: the operands are small integers
    and halves and the scales powers of two, so every sum is exact.  With
    FP4 A the last four registers of every lane hold random bytes, which must
    not matter."""
    say(f"mfma scale f8f6f4 32x32x64 layout, A format {fmt_a}")
    rng = np.random.default_rng(12 + fmt_a)
    # E4M3 bytes of the integers -16 .. 16 (and the halves -2 .. 2)
    vals = sorted({b for b in range(256) if not np.isnan(_e4m3(b)) and abs(_e4m3(b)) <= 16
                   and (2 * _e4m3(b)).is_integer()})
    b_raw = rng.choice(np.array(vals, np.uint8), size=(64, 32))
    if fmt_a == 4:
        a_raw = rng.integers(0, 256, size=(64, 32), dtype=np.uint8)
    else:
        a_raw = rng.choice(np.array(vals, np.uint8), size=(64, 32))
    # the two blocks' partial sums differ in scale by at most 2^8, so every
    # sum stays within binary32's 24 bits
    sa = rng.integers(125, 130, size=64, dtype=np.uint8)
    sb = rng.integers(125, 130, size=64, dtype=np.uint8)
    c = torch.zeros((64, 16), dtype=torch.float32, device="cuda")
    q().coli_moe_debug_mfma_f8f6f4(fmt_a, 0, torch.from_numpy(a_raw).cuda(), torch.from_numpy(b_raw).cuda(),
                                   torch.from_numpy(sa).cuda(), torch.from_numpy(sb).cuda(), c)
    got = c.cpu().numpy().astype(np.float64)
    want = _mfma_f8f6f4_model(fmt_a, a_raw, b_raw, sa, sb)
    bad = np.argwhere(got != want)
    if bad.size:
        alt = _mfma_f8f6f4_model(fmt_a, a_raw, b_raw, sa, sb, bias=8)
        unscaled = _mfma_f8f6f4_model(fmt_a, a_raw, b_raw, np.full(64, 127), np.full(64, 127))
        raise AssertionError(f"{len(bad)} lane registers differ, first {bad[:4].tolist()}: got "
                             f"{got[tuple(bad[0])]}, want {want[tuple(bad[0])]}; bias-8 model matches "
                             f"{int((got == alt).sum())}/1024, unscaled model {int((got == unscaled).sum())}/1024")


def test_mfma_fp4_times_split_activations_is_the_block_sum(torch):
    """The MXFP4 prefill product: A = a row's 32 E2M1 codes of one block in
    both scale blocks with the row's E8M0 scale x; B = the Q8_0 codes q of a
    column split as q = 16 hi + lo, E4M3 hi in the first scale block (scale
    2^4) and E4M3 lo in the second (scale 1), laid out as the kernels stage
    them.  Every result must be 2^(x - 128) * sum_j t_j q_j exactly, t_j
    twice the E2M1 value (the block sum of the MXFP4 chain)."""
    say("mfma fp4 x split activations")
    rng = np.random.default_rng(21)
    enc = {}
    for byte in range(128):
        v = _e4m3(byte)
        if float(v).is_integer() and 0 <= v <= 15:
            enc.setdefault(int(v), byte)
    for v in range(-8, 0):
        enc[v] = enc[-v] | 0x80 if -v <= 15 else None
    e2m1 = np.array([_e2m1(c) for c in range(16)])
    sb = np.concatenate([np.full(32, 131, np.uint8), np.full(32, 127, np.uint8)])
    for trial in range(8):
        codes = rng.integers(0, 16, size=(32, 32))              # [row][j]
        qv = rng.integers(-127, 128, size=(32, 32))             # [column][j]
        if trial == 0:
            codes[:] = 15                                       # -6 everywhere
            qv[:] = 127
        x = rng.integers(40, 200, size=32).astype(np.uint8)
        hi, lo = qv >> 4, qv & 15
        a = rng.integers(0, 256, size=(64, 32)).astype(np.uint8)  # bytes 16-31 unused
        b = np.zeros((64, 32), np.uint8)
        for lane in range(64):
            i, half = lane % 32, lane // 32
            a[lane, :16] = [codes[i, 2 * j] | (codes[i, 2 * j + 1] << 4) for j in range(16)]
            js = range(16 * half, 16 * half + 16)
            b[lane, :16] = [enc[int(hi[i, j])] for j in js]
            b[lane, 16:] = [enc[int(lo[i, j])] for j in js]
        c = torch.zeros((64, 16), dtype=torch.float32, device="cuda")
        q().coli_moe_debug_mfma_f8f6f4(4, 0, torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(),
                                       torch.from_numpy(np.concatenate([x, x])).cuda(), torch.from_numpy(sb).cuda(), c)
        got = c.cpu().numpy().astype(np.float64)
        isum = (2 * e2m1[codes]) @ qv.T                          # [row][column], exact integers
        C = isum * 2.0 ** (x.astype(np.float64)[:, None] - 128)
        want = np.array([[C[8 * (r // 4) + 4 * (lane // 32) + r % 4, lane % 32] for r in range(16)]
                         for lane in range(64)])
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"trial {trial}: {len(bad)} differ, first {bad[0].tolist()}: {got[tuple(bad[0])]} vs {want[tuple(bad[0])]}"


def test_roof_stream_read_reads_every_word(torch):
    """The streaming-read roof kernel really reads the whole buffer: thread g
    of the grid XOR-folds the 16-byte words g, g + T, g + 2T, ... (T threads)."""
    say("roof stream read 16 MiB")
    qm = q()
    T = qm.coli_moe_roof_sink_words()
    n16 = (16 << 20) // 16 + 5           # a ragged tail past whole grid strides
    rng = np.random.default_rng(7)
    words = rng.integers(0, 2**32, size=(n16, 4), dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32).reshape(-1)).cuda()
    sink = torch.full((T,), -1, dtype=torch.int32, device="cuda")
    qm.coli_moe_roof_stream_read(src, sink)
    got = sink.cpu().numpy().view(np.uint32)
    per_word = words[:, 0] ^ words[:, 1] ^ words[:, 2] ^ words[:, 3]
    want = np.zeros(T, np.uint32)
    for k in range(0, n16, T):
        part = per_word[k:k + T]
        want[:len(part)] ^= part
    assert np.array_equal(got, want)


def test_roof_mfma_counts_real_products(torch):
    """The int8 matrix-core roof kernel computes what its lane layout says:
    every thread's sink word is the XOR of its four chains' 16 result
    registers, each chain iters times A * B_k with A and B_k taken from the
    lanes' registers (the layout of the prefill kernels)."""
    say("roof mfma iters=3")
    qm = q()
    T = qm.coli_moe_roof_sink_words()
    iters = 3
    sink = torch.zeros((T,), dtype=torch.int32, device="cuda")
    qm.coli_moe_roof_mfma_i8(iters, sink)
    got = sink.cpu().numpy()[:256]    # every workgroup computes the same words
    want = np.zeros(256, np.int64)
    for w in range(4):
        t = 64 * w + np.arange(64)
        a = np.stack([t, t + 1, t + 2, t + 3], 1).astype(np.int32).view(np.int8).reshape(64, 16).astype(np.int64)
        l = np.arange(64)
        A = np.zeros((32, 32), np.int64)
        for j in range(16):
            A[l % 32, 16 * (l // 32) + j] = a[:, j]
        acc = np.zeros(64, np.int64)
        for k in range(4):
            bk = np.stack([3 * t + k, 5 * t + k, 7 * t + k, 11 * t + k], 1).astype(np.int32)
            bk = bk.view(np.int8).reshape(64, 16).astype(np.int64)
            B = np.zeros((32, 32), np.int64)
            for j in range(16):
                B[16 * (l // 32) + j, l % 32] = bk[:, j]
            C = (iters * (A @ B)).astype(np.int32)
            for r in range(16):
                i = 8 * (r // 4) + 4 * (l // 32) + r % 4
                acc ^= C[i, l % 32].astype(np.int64)
        want[64 * w:64 * w + 64] = acc
    assert np.array_equal(got.astype(np.int64), want.astype(np.int32).astype(np.int64))
    assert np.array_equal(sink.cpu().numpy().reshape(-1, 256), np.tile(got, (T // 256, 1)))
