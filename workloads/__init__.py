"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no attention arithmetic: it only names the workload shapes
and draws the random inputs, so that the GPU path and the CPU oracle see
exactly the same numbers.

Recipe (one stream per tensor and per (batch, head), so any head can be drawn
on its own without drawing the whole problem):

* generator: ``numpy.random.Generator(PCG64(SeedSequence([seed, t, b, h])))``
  where ``t`` is 0, 1, 2, 3 for Q, K, V, dO;
* values: ``standard_normal(float32)`` of shape (n, d), times the workload's
  Q multiplier for Q (3 for the peaky-softmax workload), else 1;
* rounding: for bf16 workloads the float32 values are rounded to bf16 with
  round-to-nearest-even and kept as float32 (exactly representable), so the
  oracle upcasts the very values the GPU receives.
* grouped-query workloads (``kv_heads`` < H): K and V are drawn for heads
  ``h < kv_heads`` only, with the same per-(b, h) streams.
* sparse-pattern workloads: global token positions are the first
  ``n_global // 2`` positions plus the rest drawn without replacement from
  the remaining positions (``SeedSequence([seed, 100])``); a BigBird layout
  ``(local, global, random)`` over 64-token blocks sets the blocks within
  ``local // 2`` of the diagonal, every block of the first ``global`` block
  rows and columns, and, in every other block row, ``random`` further blocks
  drawn without replacement from the unset ones (``SeedSequence([seed, 200,
  row])``).  The same arrays go to the GPU and to the oracle.
* FP8 rotation signs: ``+-1`` with equal probability from
  ``SeedSequence([seed, 300])``.
"""

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "VARIANTS",
    "SPARSE_IO",
    "workload",
    "round_to_bf16",
    "draw_head",
    "draw_inputs",
    "pair_count",
    "draw_pattern",
    "draw_signs",
    "pattern_pair_count",
    "LAYOUT_BLOCK",
]

TENSORS = ("q", "k", "v", "do")


@dataclass(frozen=True)
class Workload:
    """One problem shape: Q, O, dO [B, H, n, d]; K, V [B, Hkv, n, d]
    (Hkv = ``kv_heads``, 0 meaning H); element type, window."""

    name: str
    B: int
    H: int
    n: int
    d: int
    dtype: str  # "f32" or "bf16"
    window: int = -1  # -1: no mask; w >= 0: |i - j| <= w
    q_mult: float = 1.0
    seed: int = 69000
    kv_heads: int = 0  # 0: one key/value head per query head
    n_global: int = 0  # sparse pattern: number of global tokens
    bigbird: tuple = ()  # sparse pattern: (local, global, random) blocks of 64
    fp8: bool = False  # FP8 forward (E4M3 inputs quantised per head)
    rotate: bool = False  # FP8: Hadamard rotation of Q and K with drawn signs
    note: str = field(default="", compare=False)

    @property
    def has_pattern(self):
        return self.n_global > 0 or bool(self.bigbird)

    @property
    def scale(self):
        return float(1.0 / np.sqrt(self.d))

    @property
    def Hkv(self):
        return self.kv_heads or self.H

    @property
    def group(self):
        return self.H // self.Hkv

    @property
    def shape(self):
        return (self.B, self.H, self.n, self.d)

    def tensor_shape(self, tensor):
        return (self.B, self.Hkv, self.n, self.d) if tensor in ("k", "v") else self.shape


WORKLOADS = [
    Workload("single_head_f32_n256_d64", 1, 1, 256, 64, "f32", seed=69001,
             note="single head, fp32, oracle-sized"),
    Workload("bf16_b4h16_n2048_d64", 4, 16, 2048, 64, "bf16", seed=69002),
    Workload("bf16_b2h32_n8192_d128_q3", 2, 32, 8192, 128, "bf16", q_mult=3.0,
             seed=69003, note="Q scaled by 3: peaky softmax rows"),
    Workload("bf16_b1h16_n32768_d128", 1, 16, 32768, 128, "bf16", seed=69004,
             note="long context"),
    Workload("bf16_b2h8_n16384_d256_w512", 2, 8, 16384, 256, "bf16", window=512,
             seed=69005, note="Longformer-style local window |i-j|<=512"),
]

# Follow-on variants, measured beside the workloads above.
VARIANTS = [
    Workload("bf16_b2h32kv8_n8192_d128_gqa", 2, 32, 8192, 128, "bf16", seed=69006, kv_heads=8,
             note="grouped-query: 8 key/value heads, each shared by 4 query heads"),
    Workload("bf16_b1h16_n16384_d128_longformer_w256_g16", 1, 16, 16384, 128, "bf16", window=256, seed=69007,
             n_global=16, note="Longformer: window |i-j|<=256 plus 16 global tokens"),
    Workload("bf16_b1h16_n16384_d128_bigbird_b64", 1, 16, 16384, 128, "bf16", seed=69008, bigbird=(3, 2, 3),
             note="BigBird: 64-token blocks, 3 local, 2 global, 3 random per block row"),
    Workload("fp8_b2h32_n8192_d128_rot", 2, 32, 8192, 128, "bf16", seed=69009, fp8=True, rotate=True,
             note="FP8 forward: E4M3 inputs with the Hadamard rotation of Q and K"),
    Workload("fp8_b4h16_n2048_d64_rot", 4, 16, 2048, 64, "bf16", seed=69010, fp8=True, rotate=True,
             note="FP8 forward at d=64 (the 4x16-head, n=2048 shape)"),
]


# Block-sparse I/O sweep (not benchmarked by default): BigBird layouts whose
# visible pairs grow with the number of random blocks per block row at a
# fixed input size, and whose inputs grow with n at a fixed layout density.
SPARSE_IO = [
    Workload(f"bf16_b1h16_n16384_d128_bigbird_r{r}", 1, 16, 16384, 128, "bf16", seed=69008, bigbird=(3, 2, r),
             note=f"BigBird with {r} random blocks per block row")
    for r in (1, 7, 15)
] + [
    Workload(f"bf16_b1h16_n{n}_d128_bigbird_b64", 1, 16, n, 128, "bf16", seed=69008, bigbird=(3, 2, 3),
             note=f"BigBird 3/2/3 at n={n}")
    for n in (8192, 32768)
]


def draw_signs(wl, d=None):
    """The +-1 signs of the FP8 rotation (float32, d entries)."""
    d = wl.d if d is None else d
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, 300])))
    return np.where(g.random(d) < 0.5, -1.0, 1.0).astype(np.float32)

LAYOUT_BLOCK = 64


def draw_pattern(wl):
    """(window, global positions int32 sorted, layout uint8 [nb, nb] or None)
    of a sparse-pattern workload (recipe in the module docstring)."""
    n = wl.n
    glob = np.zeros(0, dtype=np.int32)
    if wl.n_global:
        head = np.arange(wl.n_global // 2)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, 100])))
        rest = g.choice(np.arange(wl.n_global // 2, n), size=wl.n_global - wl.n_global // 2, replace=False)
        glob = np.sort(np.concatenate([head, rest])).astype(np.int32)
    layout = None
    if wl.bigbird:
        local, nglob, nrand = wl.bigbird
        nb = -(-n // LAYOUT_BLOCK)
        i = np.arange(nb)
        layout = (np.abs(i[:, None] - i[None, :]) <= local // 2)
        layout[:nglob, :] = True
        layout[:, :nglob] = True
        for r in range(nglob, nb):
            free = np.flatnonzero(~layout[r])
            g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, 200, r])))
            pick = g.choice(free, size=min(nrand, free.size), replace=False)
            layout[r, pick] = True
        layout = layout.astype(np.uint8)
    return wl.window, glob, layout


def pattern_pair_count(n, window, global_idx, layout, row_block=1024):
    """Visible (query, key) pairs of a sparse pattern (for FLOP counts)."""
    isg = np.zeros(n, dtype=bool)
    isg[np.asarray(global_idx, dtype=np.int64)] = True
    cols = np.arange(n)
    total = 0
    for r0 in range(0, n, row_block):
        rows = np.arange(r0, min(n, r0 + row_block))
        vis = isg[rows][:, None] | isg[None, :]
        if window >= 0:
            vis = vis | (np.abs(rows[:, None] - cols[None, :]) <= window)
        if layout is not None:
            vis = vis | layout.astype(bool)[rows // LAYOUT_BLOCK][:, cols // LAYOUT_BLOCK]
        total += int(vis.sum())
    return total


def workload(name_or_index):
    """Look a workload up by name or by its position in ``WORKLOADS``."""
    if isinstance(name_or_index, int):
        return WORKLOADS[name_or_index]
    for w in WORKLOADS + VARIANTS + SPARSE_IO:
        if w.name == name_or_index:
            return w
    raise KeyError(name_or_index)


def round_to_bf16(x):
    """Round float32 values to the nearest bf16 (ties to even), as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(x.shape)


def _stream(seed, t, b, h):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, t, b, h])))


def draw_head(wl, tensor, b, h, n=None, d=None):
    """One (n, d) float32 slice of ``tensor`` ('q','k','v','do') at (b, h)."""
    n = wl.n if n is None else n
    d = wl.d if d is None else d
    t = TENSORS.index(tensor)
    x = _stream(wl.seed, t, b, h).standard_normal((n, d), dtype=np.float32)
    if tensor == "q" and wl.q_mult != 1.0:
        x *= np.float32(wl.q_mult)
    if wl.dtype == "bf16":
        x = round_to_bf16(x)
    return x


def draw_inputs(wl, tensors=TENSORS, heads=None):
    """Dict of float32 arrays [B, H, n, d] ([B, Hkv, n, d] for K and V; or
    [len(heads), n, d] if ``heads`` lists (b, h) pairs) for the requested
    tensors."""
    out = {}
    for name in tensors:
        if heads is None:
            shape = wl.tensor_shape(name)
            arr = np.empty(shape, dtype=np.float32)
            for b in range(shape[0]):
                for h in range(shape[1]):
                    arr[b, h] = draw_head(wl, name, b, h)
        else:
            arr = np.stack([draw_head(wl, name, b, h) for (b, h) in heads])
        out[name] = arr
    return out


def pair_count(n, window):
    """Number of (query, key) pairs that take part: n*n without a window,
    else the pairs with |i - j| <= window."""
    if window < 0 or window >= n - 1:
        return n * n
    w = window
    return n * (2 * w + 1) - w * (w + 1)
