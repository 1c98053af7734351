"""Seeded synthetic inputs for the routed-expert MoE layer.

This module only produces input bytes: hidden states, the router gate and
bias, and expert weight blobs in the packed layout.  It holds none of the
layer's own arithmetic (no activation quantisation, no routing, no expert
FFN, no combine); the CPU oracle and the HIP library each consume exactly the
bytes written here.  Routing-shaping constructions use only library linear
algebra and sorting on target logits, never the layer's router.

Random numbers come from SplitMix64 (Steele, Lea & Flood, OOPSLA 2014) used
as a counter-based generator: value i of stream `key` is
mix64(key + (i + 1) * GAMMA), and keys are derived by folding
(seed, kind, indices...) through mix64.  The C helper `gen.c` implements the
same stream for the large blobs.

Two weight recipes:
  * gaussian: w ~ N(0, sigma) per element (Box-Muller on the stream), then
    the offline per-row quantiser (amax / qmax scale, round half away from
    zero, clamp).  Used for small layers, where it is cheap.
  * cdf: codes drawn i.i.d. from the distribution of that quantised Gaussian
    (a 65536-entry inverse-CDF table with a nominal amax of 4 sigma), with a
    per-row scale jittered +-5% around the nominal one.  Used for
    GLM-5.2-shaped layers, where tens of gigabytes must be written quickly.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
MASK64 = (1 << 64) - 1

# stream kinds
K_X = 1
K_ROUTER_W = 2
K_ROUTER_BIAS = 3
K_WEIGHT = 4
K_ROUTING = 5

QRANGE = {8: (-127, 127), 4: (-7, 7), 2: (-2, 1)}
QMAX = {8: 127, 4: 7, 2: 2}


# --------------------------------------------------------------------------
# counter-based random streams
# --------------------------------------------------------------------------
def _mix64_int(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def _mix64(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    z ^= z >> np.uint64(30)
    z *= np.uint64(0xBF58476D1CE4E5B9)
    z ^= z >> np.uint64(27)
    z *= np.uint64(0x94D049BB133111EB)
    z ^= z >> np.uint64(31)
    return z


def stream_key(seed: int, *parts: int) -> int:
    """Folds (seed, parts...) into one 64-bit stream key."""
    k = _mix64_int(seed + GAMMA)
    for p in parts:
        k = _mix64_int(k ^ _mix64_int((p & MASK64) + GAMMA))
    return k


def uniform_u64(key: int, n: int, offset: int = 0) -> np.ndarray:
    """Values offset..offset+n-1 of the stream `key` as uint64."""
    i = np.arange(offset + 1, offset + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + i * np.uint64(GAMMA)
    return _mix64(z)


def uniform01(key: int, n: int, offset: int = 0) -> np.ndarray:
    """Uniform doubles in [0, 1) with 53 random bits."""
    return (uniform_u64(key, n, offset) >> np.uint64(11)).astype(np.float64) * 2.0**-53


def normal(key: int, n: int) -> np.ndarray:
    """n standard normals (f64); value i uses stream values 2i and 2i+1."""
    r = uniform_u64(key, 2 * n).reshape(n, 2)
    u1 = ((r[:, 0] >> np.uint64(11)).astype(np.float64) + 0.5) * 2.0**-53
    u2 = (r[:, 1] >> np.uint64(11)).astype(np.float64) * 2.0**-53
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)


# --------------------------------------------------------------------------
# layer shapes
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class LayerSpec:
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    n_shared: int
    wbits: int
    routed_scaling_factor: float = 2.5
    norm_topk_prob: int = 1
    group: int = 0          # 0: one scale per row; 64: one per 64 codes of a row
    fmt: int = 0            # 0: integer codes; 1: MXFP4 (E2M1 codes, one E8M0 scale per 32)

    @property
    def blob_bytes(self) -> int:
        return blob_layout(self.hidden, self.inter, self.wbits, self.group, self.fmt)["total"]


TINY = LayerSpec(hidden=256, inter=128, n_experts=16, top_k=2, n_shared=1, wbits=4)
GLM = LayerSpec(hidden=6144, inter=2048, n_experts=256, top_k=8, n_shared=1, wbits=4)
GLM_INT8 = dataclasses.replace(GLM, wbits=8)
GLM_INT2 = dataclasses.replace(GLM, wbits=2)
TINY_GS64 = dataclasses.replace(TINY, group=64)
GLM_GS64 = dataclasses.replace(GLM, group=64)
TINY_MX = dataclasses.replace(TINY, fmt=1)
GLM_MX = dataclasses.replace(GLM, fmt=1)


def blob_layout(hidden: int, inter: int, bits: int, group: int = 0, fmt: int = 0) -> dict:
    """Byte offsets of the six sections of one expert blob.

    [gate codes: inter rows x hidden*bits/8][up codes: same][down codes:
    hidden rows x inter*bits/8][gate scales f32 x inter][up scales f32 x
    inter][down scales f32 x hidden]; every section starts on a 256-byte
    boundary and the total is rounded up to 256 bytes.  With group > 0 the
    scale sections hold one f32 per `group` codes of a row, row-major:
    [inter][hidden/group], [inter][hidden/group], [hidden][inter/group].
    """
    a = lambda n: (n + 255) // 256 * 256  # noqa: E731
    gate = inter * hidden * bits // 8
    down = hidden * inter * bits // 8
    sgu = 4 * inter * (hidden // group if group else 1)
    sd = 4 * hidden * (inter // group if group else 1)
    if fmt == 1:   # MXFP4: 4-bit codes, one E8M0 byte per 32 codes of a row
        gate, down = inter * hidden // 2, hidden * inter // 2
        sgu, sd = inter * (hidden // 32), hidden * (inter // 32)
    off = {"gate": 0}
    off["up"] = a(gate)
    off["down"] = a(off["up"] + gate)
    off["s_gate"] = a(off["down"] + down)
    off["s_up"] = a(off["s_gate"] + sgu)
    off["s_down"] = a(off["s_up"] + sgu)
    off["total"] = a(off["s_down"] + sd)
    return off


# --------------------------------------------------------------------------
# offline weight quantiser and packer (data preparation, not the layer)
# --------------------------------------------------------------------------
def _round_half_away(v: np.ndarray) -> np.ndarray:
    return np.sign(v) * np.floor(np.abs(v) + 0.5)


def quantize_rows(w: np.ndarray, bits: int) -> tuple[np.ndarray, np.ndarray]:
    """Per-row symmetric quantiser: scale = amax/qmax, code = clamp(round(w/scale))."""
    lo, hi = QRANGE[bits]
    w = np.asarray(w, dtype=np.float64)
    amax = np.max(np.abs(w), axis=1)
    s = (amax / QMAX[bits]).astype(np.float32)
    s64 = s.astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s64[:, None] > 0, _round_half_away(w / s64[:, None]), 0.0)
    q = np.clip(q, lo, hi).astype(np.int8)
    return q, s


def quantize_groups(w: np.ndarray, bits: int, group: int) -> tuple[np.ndarray, np.ndarray]:
    """quantize_rows applied to every `group` consecutive weights of a row:
    codes [rows, cols], scales [rows, cols / group]."""
    rows, cols = w.shape
    q, s = quantize_rows(np.asarray(w).reshape(rows * (cols // group), group), bits)
    return q.reshape(rows, cols), s.reshape(rows, cols // group)


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Packs signed codes [rows, cols] into the blob byte layout.

    Per 32-element block: int8 -> 32 bytes as is; int4 -> 16 bytes, byte j
    holds element j in bits 0-3 and element j+16 in bits 4-7; int2 -> 8
    bytes, byte j holds element j+8i in bits 2i..2i+1 (i = 0..3).  Codes are
    stored in two's complement.
    """
    codes = np.asarray(codes, dtype=np.int8)
    rows, cols = codes.shape
    assert cols % 32 == 0
    blk = codes.reshape(rows, cols // 32, 32).view(np.uint8)
    if bits == 8:
        return blk.reshape(rows, cols).copy()
    if bits == 4:
        lo = blk[:, :, :16] & 0x0F
        hi = (blk[:, :, 16:] & 0x0F) << 4
        return (lo | hi).astype(np.uint8).reshape(rows, cols // 2)
    if bits == 2:
        out = np.zeros((rows, cols // 32, 8), dtype=np.uint8)
        for i in range(4):
            out |= ((blk[:, :, 8 * i:8 * i + 8] & 0x03) << (2 * i)).astype(np.uint8)
        return out.reshape(rows, cols // 4)
    raise ValueError(bits)


def assemble_blob(hidden, inter, bits, gate_codes, up_codes, down_codes, s_gate, s_up, s_down, group=0):
    lay = blob_layout(hidden, inter, bits, group)
    blob = np.zeros(lay["total"], dtype=np.uint8)

    def put(name, arr):
        b = np.ascontiguousarray(arr).view(np.uint8).ravel()
        blob[lay[name]:lay[name] + b.size] = b

    put("gate", pack_codes(gate_codes, bits))
    put("up", pack_codes(up_codes, bits))
    put("down", pack_codes(down_codes, bits))
    put("s_gate", np.asarray(s_gate, np.float32))
    put("s_up", np.asarray(s_up, np.float32))
    put("s_down", np.asarray(s_down, np.float32))
    return blob


def gaussian_expert(seed: int, layer: int, expert: int, spec: LayerSpec, sigma: float = 0.02):
    """Expert weights w ~ N(0, sigma), per-row (or, with spec.group, per
    row-group) quantised.

    Returns (blob, parts) where parts holds the codes and scales of the
    three matrices (gate/up [inter, hidden], down [hidden, inter]).
    """
    H, I, b, G = spec.hidden, spec.inter, spec.wbits, spec.group
    parts = {}
    for m, (name, rows, cols) in enumerate((("gate", I, H), ("up", I, H), ("down", H, I))):
        key = stream_key(seed, K_WEIGHT, layer, expert, m)
        w = (normal(key, rows * cols) * sigma).astype(np.float32).reshape(rows, cols)
        q, s = quantize_groups(w, b, G) if G else quantize_rows(w, b)
        parts[name] = q
        parts["s_" + name] = s
    blob = assemble_blob(H, I, b, parts["gate"], parts["up"], parts["down"],
                         parts["s_gate"], parts["s_up"], parts["s_down"], G)
    return blob, parts


# --------------------------------------------------------------------------
# MXFP4 experts (offline quantiser and packer; data preparation only)
# --------------------------------------------------------------------------
# magnitudes of the E2M1 codes 0..7 (code 8 + m is the negative of code m)
E2M1_MAG = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def e2m1_round(x: np.ndarray) -> np.ndarray:
    """E2M1 code (0..15) nearest to each value (ties to the even magnitude
    index), saturating at +-6."""
    x = np.asarray(x, np.float64)
    mag = np.asarray(E2M1_MAG)
    a = np.minimum(np.abs(x), 6.0)
    d = np.abs(a[..., None] - mag)
    best = np.argmin(d + 1e-12 * (np.arange(8) % 2), axis=-1)
    return (best + np.where((x < 0) & (best > 0), 8, 0)).astype(np.uint8)


def quantize_mx_rows(w: np.ndarray):
    """MXFP4 quantiser (OCP Microscaling): per 32 values of a row, the shared
    exponent floor(log2(amax)) - 2 (6 = 1.5 * 2^2 is the largest element),
    E8M0 byte = exponent + 127 clamped to [0, 254] (0 when amax is 0), codes
    the nearest E2M1 of w / 2^exponent.  Returns (codes [rows, cols] 0..15,
    scale bytes [rows, cols / 32])."""
    w = np.asarray(w, np.float64)
    rows, cols = w.shape
    wb = w.reshape(rows, cols // 32, 32)
    amax = np.abs(wb).max(-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    xb = np.clip(e + 127, 0, 254).astype(np.uint8)
    codes = e2m1_round(wb / np.exp2(xb.astype(np.float64) - 127)[..., None])
    return codes.reshape(rows, cols), xb


def pack_mx(codes: np.ndarray) -> np.ndarray:
    """Two E2M1 codes per byte: element 2j in bits 0-3, element 2j+1 in bits 4-7."""
    c = np.asarray(codes, np.uint8)
    return (c[:, 0::2] & 0x0F) | ((c[:, 1::2] & 0x0F) << 4)


def assemble_mx_blob(hidden, inter, gate_codes, up_codes, down_codes, x_gate, x_up, x_down):
    lay = blob_layout(hidden, inter, 4, 0, 1)
    blob = np.zeros(lay["total"], dtype=np.uint8)
    for name, arr in (("gate", pack_mx(gate_codes)), ("up", pack_mx(up_codes)), ("down", pack_mx(down_codes)),
                      ("s_gate", x_gate), ("s_up", x_up), ("s_down", x_down)):
        b = np.ascontiguousarray(arr, dtype=np.uint8).ravel()
        blob[lay[name]:lay[name] + b.size] = b
    return blob


def mx_expert(seed: int, layer: int, expert: int, spec: LayerSpec, sigma: float = 0.02):
    """MXFP4 expert: w ~ N(0, sigma) quantised by quantize_mx_rows.
    Returns (blob, parts) with the codes and scale bytes of each matrix."""
    H, I = spec.hidden, spec.inter
    parts = {}
    for m, (name, rows, cols) in enumerate((("gate", I, H), ("up", I, H), ("down", H, I))):
        key = stream_key(seed, K_WEIGHT, layer, expert, m)
        w = (normal(key, rows * cols) * sigma).reshape(rows, cols)
        parts[name], parts["s_" + name] = quantize_mx_rows(w)
    blob = assemble_mx_blob(H, I, parts["gate"], parts["up"], parts["down"],
                            parts["s_gate"], parts["s_up"], parts["s_down"])
    return blob, parts


def extreme_mx_parts(seed: int, layer: int, expert: int, spec: LayerSpec) -> dict:
    """Edge-case MXFP4 codes and scales: every code 0..15 (the negative zero
    8 and both ends +-6 included) at every position of a block (row r holds
    code (j + r) % 16 at position j), with rows 32..63 of gate and up equal
    and at -6 throughout (h constant over that block, so Q8_0(h) is +-127);
    scale bytes drawn from 0, 1, 2 (subnormal and smallest normal
    multipliers), 100, 120, 127 and 130, one common byte per flat row."""
    H, I = spec.hidden, spec.inter
    choices = np.array([0, 1, 2, 100, 120, 127, 130], np.uint8)
    parts = {}
    for m, (name, rows, cols) in enumerate((("gate", I, H), ("up", I, H), ("down", H, I))):
        c = ((np.arange(cols)[None, :] + np.arange(rows)[:, None]) % 16).astype(np.uint8)
        u = uniform_u64(stream_key(seed, K_WEIGHT, layer, expert, m, 9), rows * (cols // 32))
        x = choices[(u % np.uint64(len(choices))).astype(np.int64)].reshape(rows, cols // 32)
        if name != "down" and rows >= 64:
            c[32:64] = 15
            x[32:64] = x[32, 0]
        parts[name], parts["s_" + name] = c, x
    return parts


def extreme_mx_layer(seed: int, S: int, spec: LayerSpec, layer: int = 0) -> dict:
    """A small MXFP4 layer of extreme_mx_parts blobs with extreme_hidden_states."""
    blobs = []
    for e in range(spec.n_experts + spec.n_shared):
        p = extreme_mx_parts(seed, layer, e, spec)
        blobs.append(assemble_mx_blob(spec.hidden, spec.inter, p["gate"], p["up"], p["down"],
                                      p["s_gate"], p["s_up"], p["s_down"]))
    return {
        "spec": spec,
        "x": extreme_hidden_states(seed, layer, S, spec.hidden),
        "router_w": router_weights(seed, layer, spec),
        "bias": router_bias(seed, layer, spec),
        "blobs": blobs[:spec.n_experts],
        "shared": blobs[spec.n_experts] if spec.n_shared else None,
    }


def mx_cdf_table(ratio: float = 2.56) -> np.ndarray:
    """65536-entry table mapping a 16-bit uniform to an E2M1 code, distributed
    as the nearest E2M1 of z * ratio for z ~ N(0, 1) (ratio: the weights'
    standard deviation over the block scale; 0.02 / 2^-7 by default)."""
    mag = np.asarray(E2M1_MAG)
    mids = (mag[:-1] + mag[1:]) / 2                     # thresholds between magnitudes
    # P(|x| < mid_k), x = z * ratio
    cdf_abs = np.array([math.erf(t / ratio / math.sqrt(2.0)) for t in mids])
    probs = np.diff(np.concatenate([[0.0], cdf_abs, [1.0]]))   # magnitude 0..7
    # signed codes: magnitude 0 once (code 0), others split evenly by sign
    p = np.zeros(16)
    p[0] = probs[0]
    p[1:8] = probs[1:] / 2
    p[9:16] = probs[1:] / 2
    edges = np.round(np.cumsum(p) * 65536.0).astype(np.int64)
    u = np.arange(65536)
    idx = np.searchsorted(edges, u, side="right")
    return np.minimum(idx, 15).astype(np.uint8)


def mx_cdf_expert_into(out_ptr: int, seed: int, layer: int, expert: int, spec: LayerSpec,
                       threads: int | None = None) -> int:
    """Writes one GLM-sized MXFP4 blob (codes from mx_cdf_table, E8M0 scale
    bytes uniform over 119..121) at host address out_ptr; returns its size."""
    lib = _load()
    table = mx_cdf_table()
    keys = (ctypes.c_uint64 * 6)(*[stream_key(seed, K_WEIGHT, layer, expert, m, part, 11)
                                   for m in range(3) for part in (0, 1)])
    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    n = lib.synth_fill_blob_mx(keys, spec.hidden, spec.inter, table.ctypes.data, 119, 3, out_ptr, threads)
    if n != spec.blob_bytes:
        raise RuntimeError("synth_fill_blob_mx rejected the shape")
    return int(n)


# --------------------------------------------------------------------------
# edge-case inputs: the code range's extremes
# --------------------------------------------------------------------------
# every code the formats admit, the minimum included (the quantisers above
# never produce int4 -8 or int8 -128, but the blob format holds them)
FULL_RANGE = {8: (-128, 127), 4: (-8, 7), 2: (-2, 1)}


def extreme_codes(key: int, rows: int, cols: int, bits: int, flat_rows: tuple = ()) -> np.ndarray:
    """Codes [rows, cols] built around the range's minimum lo and maximum hi:
    row r % 4 == 0 holds lo at position (r // 4) % 32 of every 32-code block
    and hi elsewhere, r % 4 == 2 the same at position (r // 4 + 16) % 32 (so
    that every position gets the minimum alone in some row of any matrix of
    at least 64 rows outside flat_rows); r % 4 == 1 is lo everywhere; r % 4
    == 3 alternates lo and hi when r // 4 is even and is uniform over the
    whole range when it is odd.  Rows in flat_rows (a range) are lo
    everywhere, so that their dot products with one vector are equal."""
    lo, hi = FULL_RANGE[bits]
    u = uniform_u64(key, rows * cols).reshape(rows, cols)
    codes = (lo + (u % np.uint64(hi - lo + 1)).astype(np.int64)).astype(np.int8)
    pos = np.arange(cols) % 32
    for r in range(rows):
        m, j = r % 4, r // 4
        if m == 0:
            codes[r] = np.where(pos == j % 32, lo, hi)
        elif m == 2:
            codes[r] = np.where(pos == (j + 16) % 32, lo, hi)
        elif m == 1:
            codes[r] = lo
        elif j % 2 == 0:
            codes[r] = np.where(pos % 2 == 0, lo, hi)
    if flat_rows:
        codes[flat_rows[0]:flat_rows[1]] = lo
    return codes


def extreme_parts(seed: int, layer: int, expert: int, spec: LayerSpec) -> dict:
    """Codes and scales of an edge-case expert (see extreme_expert)."""
    H, I, b, G = spec.hidden, spec.inter, spec.wbits, spec.group
    flat = (32, 64) if I >= 64 else ()
    parts = {}
    for m, (name, rows, cols) in enumerate((("gate", I, H), ("up", I, H), ("down", H, I))):
        key = stream_key(seed, K_WEIGHT, layer, expert, m, 7)
        parts[name] = extreme_codes(key, rows, cols, b, flat if name != "down" else ())
        ns = cols // G if G else 1
        s = (0.0025 + 0.005 * uniform01(stream_key(seed, K_WEIGHT, layer, expert, m, 8), rows * ns))
        s = s.astype(np.float32).reshape(rows, ns)
        if flat and name != "down":
            s[flat[0]:flat[1]] = s[flat[0]]
        parts["s_" + name] = s if G else s[:, 0].copy()
    return parts


def extreme_expert(seed: int, layer: int, expert: int, spec: LayerSpec) -> np.ndarray:
    """A blob whose codes come from extreme_codes: gate and up rows 32..63
    are all lo with one common scale, so that a token's h is the same over
    that block of 32 and its Q8_0 codes are all +-127; scales (per row or per
    group) are seeded uniforms in [0.0025, 0.0075)."""
    p = extreme_parts(seed, layer, expert, spec)
    return assemble_blob(spec.hidden, spec.inter, spec.wbits, p["gate"], p["up"], p["down"],
                         p["s_gate"], p["s_up"], p["s_down"], spec.group)


def extreme_hidden_states(seed: int, layer: int, S: int, H: int) -> np.ndarray:
    """x [S, H] f32 whose 32-value blocks each hold one magnitude (a seeded
    uniform in [0.5, 2)), so that every Q8_0 code is +-127: block b of a
    token is all positive when (b + t) % 3 == 0, all negative when it is 1,
    and of seeded random signs when it is 2."""
    nb = H // 32
    mag = 0.5 + 1.5 * uniform01(stream_key(seed, K_X, layer, 900), S * nb).reshape(S, nb)
    rnd = uniform01(stream_key(seed, K_X, layer, 901), S * H).reshape(S, nb, 32) < 0.5
    mode = (np.arange(nb)[None, :] + np.arange(S)[:, None]) % 3
    sign = np.where(mode[:, :, None] == 0, 1.0, np.where(mode[:, :, None] == 1, -1.0, np.where(rnd, 1.0, -1.0)))
    return (sign * mag[:, :, None]).reshape(S, H).astype(np.float32)


def extreme_layer(seed: int, S: int, spec: LayerSpec, layer: int = 0) -> dict:
    """A small layer of extreme_expert blobs and extreme_hidden_states (router
    gate and bias as tiny_layer)."""
    blobs = [extreme_expert(seed, layer, e, spec) for e in range(spec.n_experts + spec.n_shared)]
    return {
        "spec": spec,
        "x": extreme_hidden_states(seed, layer, S, spec.hidden),
        "router_w": router_weights(seed, layer, spec),
        "bias": router_bias(seed, layer, spec),
        "blobs": blobs[:spec.n_experts],
        "shared": blobs[spec.n_experts] if spec.n_shared else None,
    }


# --------------------------------------------------------------------------
# fast large-blob recipe (C helper)
# --------------------------------------------------------------------------
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_build", "libsynth.so")
_lib = None


def build_lib(force: bool = False) -> str:
    """Compiles gen.c into synth/_build/libsynth.so."""
    if force or not os.path.exists(_LIB_PATH):
        os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               os.path.join(_HERE, "gen.c"), "-o", tmp])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build_lib())
        lib.synth_fill_blob_cdf_g.restype = ctypes.c_uint64
        lib.synth_fill_blob_cdf_g.argtypes = [
            ctypes.POINTER(ctypes.c_uint64), ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_float, ctypes.c_float, ctypes.c_void_p, ctypes.c_int]
        lib.synth_fill_blob_mx.restype = ctypes.c_uint64
        lib.synth_fill_blob_mx.argtypes = [
            ctypes.POINTER(ctypes.c_uint64), ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
        _lib = lib
    return _lib


def _phi(z: float) -> float:
    return 0.5 * (1.0 + math.erf(z / math.sqrt(2.0)))


_TABLES: dict = {}


def cdf_table(bits: int, amax_sigmas: float = 4.0) -> np.ndarray:
    """65536-entry table mapping a 16-bit uniform to a code, distributed as
    round(w/s) for w ~ N(0,1) and s = amax_sigmas/qmax, clamped to the code range."""
    if bits in _TABLES:
        return _TABLES[bits]
    lo, hi = QRANGE[bits]
    s = amax_sigmas / QMAX[bits]
    ks = np.arange(lo, hi + 1)
    upper = np.array([_phi((k + 0.5) * s) if k < hi else 1.0 for k in ks])
    thresholds = np.round(upper * 65536.0).astype(np.int64)
    u = np.arange(65536)
    idx = np.searchsorted(thresholds, u, side="right")
    table = (lo + np.minimum(idx, len(ks) - 1)).astype(np.int8)
    _TABLES[bits] = table
    return table


def cdf_expert_into(out_ptr: int, seed: int, layer: int, expert: int, spec: LayerSpec,
                    sigma: float = 0.02, threads: int | None = None) -> int:
    """Writes one cdf-recipe blob at host address out_ptr; returns its size."""
    lib = _load()
    table = cdf_table(spec.wbits)
    keys = (ctypes.c_uint64 * 6)(*[stream_key(seed, K_WEIGHT, layer, expert, m, part)
                                   for m in range(3) for part in (0, 1)])
    nominal = 4.0 * sigma / QMAX[spec.wbits]
    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    n = lib.synth_fill_blob_cdf_g(keys, spec.hidden, spec.inter, spec.wbits, spec.group,
                                  table.ctypes.data, nominal, 0.1, out_ptr, threads)
    if n != spec.blob_bytes:
        raise RuntimeError("synth_fill_blob_cdf rejected the shape")
    return int(n)


def cdf_expert(seed: int, layer: int, expert: int, spec: LayerSpec, sigma: float = 0.02) -> np.ndarray:
    blob = np.empty(spec.blob_bytes, dtype=np.uint8)
    if spec.fmt == 1:
        mx_cdf_expert_into(blob.ctypes.data, seed, layer, expert, spec)
    else:
        cdf_expert_into(blob.ctypes.data, seed, layer, expert, spec, sigma)
    return blob


def expert_blob(seed: int, layer: int, expert: int, spec: LayerSpec) -> np.ndarray:
    """The blob of routed expert `expert` (or the shared expert, expert ==
    n_experts) of `layer`, with the recipe chosen by size."""
    if spec.hidden * spec.inter <= 1 << 20:
        if spec.fmt == 1:
            return mx_expert(seed, layer, expert, spec)[0]
        return gaussian_expert(seed, layer, expert, spec)[0]
    return cdf_expert(seed, layer, expert, spec)


# --------------------------------------------------------------------------
# hidden states, router gate and bias
# --------------------------------------------------------------------------
def router_weights(seed: int, layer: int, spec: LayerSpec) -> np.ndarray:
    """W_r [E, H] f32 ~ N(0, 1/H) so that logits are about N(0, 1)."""
    key = stream_key(seed, K_ROUTER_W, layer)
    w = normal(key, spec.n_experts * spec.hidden) / math.sqrt(spec.hidden)
    return w.astype(np.float32).reshape(spec.n_experts, spec.hidden)


def router_bias(seed: int, layer: int, spec: LayerSpec, std: float = 0.01) -> np.ndarray:
    key = stream_key(seed, K_ROUTER_BIAS, layer)
    return (normal(key, spec.n_experts) * std).astype(np.float32)


def hidden_states(seed: int, layer: int, S: int, H: int, stream: int = 0) -> np.ndarray:
    """x [S, H] f32 ~ N(0, 1)."""
    key = stream_key(seed, K_X, layer, stream)
    return normal(key, S * H).astype(np.float32).reshape(S, H)


def shaped_hidden_states(W_r: np.ndarray, target_logits: np.ndarray, seed: int, layer: int,
                         stream: int = 0) -> np.ndarray:
    """x [S, H] with W_r @ x_t = target_logits[t] (the minimum-norm solution,
    f64) plus N(0,1) noise projected onto the null space of W_r; stored as
    f32.

    Lets a test or benchmark fix which experts a token prefers without
    evaluating the layer's router: with zero bias the sigmoid is monotone,
    so the top-k of the target logits is the intended selection.  W_r has
    full row rank (E < H, Gaussian), so the pseudo-inverse is
    W^T (W W^T)^-1, applied through one E x E solve."""
    W = W_r.astype(np.float64)
    S = target_logits.shape[0]
    H = W.shape[1]
    z = normal(stream_key(seed, K_ROUTING, layer, stream), S * H).reshape(S, H)
    G = W @ W.T                                  # [E, E]
    rhs = target_logits.astype(np.float64).T - W @ z.T
    x = z + (W.T @ np.linalg.solve(G, rhs)).T   # z - P z + W^+ t
    return x.astype(np.float32)


def tiny_layer(seed: int = 0, S: int = 4, spec: LayerSpec = TINY, layer: int = 0) -> dict:
    """All inputs of one small layer (gaussian recipe; MXFP4 quantiser for
    spec.fmt == 1)."""
    make = mx_expert if spec.fmt == 1 else gaussian_expert
    blobs = [make(seed, layer, e, spec)[0] for e in range(spec.n_experts + spec.n_shared)]
    return {
        "spec": spec,
        "x": hidden_states(seed, layer, S, spec.hidden),
        "router_w": router_weights(seed, layer, spec),
        "bias": router_bias(seed, layer, spec),
        "blobs": blobs[:spec.n_experts],
        "shared": blobs[spec.n_experts] if spec.n_shared else None,
    }


def layer_inputs(seed: int, layer: int, spec: LayerSpec, S: int, x_stream: int = 0) -> dict:
    """Hidden states, router gate and bias of one layer (blobs not included:
    use expert_blob / cdf_expert_into for the experts that are needed)."""
    return {
        "spec": spec,
        "x": hidden_states(seed, layer, S, spec.hidden, x_stream),
        "router_w": router_weights(seed, layer, spec),
        "bias": router_bias(seed, layer, spec),
    }


def zipf_target_logits(seed: int, layer: int, spec: LayerSpec, S: int, exponent: float = 1.1,
                       batch: int = 0) -> np.ndarray:
    """Target router logits [S, E] (f64) for a Zipf-skewed prefill batch.

    Expert popularity p_e is proportional to rank^-exponent, the ranks being
    a seeded permutation of the expert ids; token t's targets are
    log p + Gumbel(0, 1) noise, so that the top-K of a row is a draw of K
    experts without replacement with probabilities proportional to p
    (the Gumbel-top-k construction).  `batch` selects an independent draw of
    the noise (same popularity)."""
    E = spec.n_experts
    perm = np.argsort(uniform01(stream_key(seed, K_ROUTING, layer, 200), E), kind="stable")
    rank = np.empty(E, np.int64)
    rank[perm] = np.arange(1, E + 1)
    logp = -exponent * np.log(rank.astype(np.float64))
    logp -= np.log(np.sum(np.exp(logp)))
    u = uniform01(stream_key(seed, K_ROUTING, layer, 201, batch), S * E).reshape(S, E)
    u = np.clip(u, 1e-300, 1.0 - 1e-16)
    gumbel = -np.log(-np.log(u))
    return logp[None, :] + gumbel


def prefill_hidden_states(seed: int, layer: int, spec: LayerSpec, S: int, exponent: float = 1.1,
                          batch: int = 0) -> np.ndarray:
    """Hidden states [S, H] f32 whose router logits are the Zipf targets of
    zipf_target_logits (pseudo-inverse construction of
    shaped_hidden_states; with zero router bias the sigmoid router then
    selects the Gumbel-top-K)."""
    W = router_weights(seed, layer, spec)
    return shaped_hidden_states(W, zipf_target_logits(seed, layer, spec, S, exponent, batch), seed, layer,
                                stream=7 + batch)


def reuse_trace(seed: int, layer: int, spec: LayerSpec, steps: int, reuse: float = 0.6) -> np.ndarray:
    """Expert sets [steps, K] of one layer over decode steps: slot k keeps the
    previous step's expert of slot k with probability `reuse` (when no
    earlier slot of the step took it), else draws uniformly from the experts
    outside the previous step's set and the step's earlier picks."""
    E, K = spec.n_experts, spec.top_k
    u = uniform01(stream_key(seed, K_ROUTING, layer, 300), steps * K * 2).reshape(steps, K, 2)
    out = np.zeros((steps, K), np.int64)
    prev: list[int] = []
    for s in range(steps):
        cur: list[int] = []
        for k in range(K):
            if prev and u[s, k, 0] < reuse and prev[k] not in cur:
                cur.append(prev[k])
                continue
            pool = [e for e in range(E) if e not in cur and e not in prev]
            cur.append(pool[int(u[s, k, 1] * len(pool))])
        out[s] = cur
        prev = cur
    return out


def trace_target_logits(seed: int, layer: int, spec: LayerSpec, trace: np.ndarray) -> np.ndarray:
    """Target logits [steps, E] whose top-K is the trace's set: the set's
    experts at 4.0, 3.75, ... in slot order, the others N(-2, 0.5)."""
    steps, K = trace.shape
    t = -2.0 + 0.5 * normal(stream_key(seed, K_ROUTING, layer, 301), steps * spec.n_experts).reshape(steps, -1)
    for k in range(K):
        t[np.arange(steps), trace[:, k]] = 4.0 - 0.25 * k
    return t


def predicted_sets(seed: int, layer: int, spec: LayerSpec, truth: np.ndarray, recall: float = 0.716) -> np.ndarray:
    """A prediction [steps, K] of the expert sets `truth` [steps, K]: slot k
    keeps the true expert with probability `recall`, else takes an expert
    drawn uniformly from those outside the true set and the step's earlier
    picks (so the expected overlap is recall * K)."""
    steps, K = truth.shape
    E = spec.n_experts
    u = uniform01(stream_key(seed, K_ROUTING, layer, 400), steps * K * 2).reshape(steps, K, 2)
    out = np.zeros((steps, K), np.int64)
    for s in range(steps):
        tset = set(int(e) for e in truth[s])
        cur: list[int] = []
        for k in range(K):
            if u[s, k, 0] < recall:
                cur.append(int(truth[s, k]))
                continue
            pool = [e for e in range(E) if e not in tset and e not in cur]
            cur.append(pool[int(u[s, k, 1] * len(pool))])
        out[s] = cur
    return out


def lookahead_hidden_states(W_here: np.ndarray, W_next: np.ndarray, t_here: np.ndarray, t_next: np.ndarray,
                            seed: int, layer: int, stream: int = 0) -> np.ndarray:
    """x [S, H] with W_here x_t = t_here[t] and W_next x_t = t_next[t] (the
    minimum-norm solution of the stacked system, f64) plus N(0,1) noise
    projected onto the null space of both gates; stored as f32.  With zero
    bias the layer's router then picks the top-K of t_here, and the next
    layer's router applied to this layer's state picks the top-K of t_next
    (a look-ahead prediction of chosen quality)."""
    W = np.concatenate([W_here, W_next]).astype(np.float64)
    t = np.concatenate([t_here, t_next], axis=1)
    return shaped_hidden_states(W, t, seed, layer, stream)


def verify_hidden_states(seed: int, layer: int, spec: LayerSpec, S: int, union_frac: float = 0.6,
                         batch: int = 0, W: np.ndarray | None = None) -> np.ndarray:
    """Hidden states of S tokens that share experts: x_t = sqrt(rho) c +
    sqrt(1 - rho) n_t with a common direction c, rho bisected so that the
    top-K sets of the logits W_r x_t cover about union_frac * S * K distinct
    experts.  Uses float64 logits and a sort only (bias ignored); the realised
    union of the actual router is reported by whoever routes these tokens.
    `batch` selects an independent draw; W (the layer's router gate) may be
    passed to skip regenerating it."""
    if W is None:
        W = router_weights(seed, layer, spec)
    W = W.astype(np.float64)
    H, K = spec.hidden, spec.top_k
    extra = (batch,) if batch else ()
    c = normal(stream_key(seed, K_ROUTING, layer, 100, *extra), H)
    n = normal(stream_key(seed, K_ROUTING, layer, 101, *extra), S * H).reshape(S, H)
    lc, ln = W @ c, n @ W.T

    def make(rho):
        return math.sqrt(rho) * c[None, :] + math.sqrt(1.0 - rho) * n

    def union(rho):
        top = np.argsort(-(math.sqrt(rho) * lc[None, :] + math.sqrt(1.0 - rho) * ln), axis=1, kind="stable")[:, :K]
        return len(set(top.ravel().tolist())) / (S * K)

    lo, hi = 0.0, 1.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        if union(mid) > union_frac:
            lo = mid
        else:
            hi = mid
    return make(hi).astype(np.float32)
