"""Seeded synthetic workloads: op queues plus the initial contents of their buffers.

This module only *describes* queues of small tensor ops and draws their inputs.
It performs none of the ops' arithmetic: the CPU oracle (under ``oracle/``) and
the HIP runtime (through :mod:`persistent_fusion_amd.gpuos`) both consume the
same :class:`Workload` and compute the results independently.

Input recipe (documented once here, used by every generator):

* random numbers come from ``numpy.random.default_rng(seed)`` (PCG64), one
  generator per workload, drawn in a fixed order;
* U(-1, 1) values are ``k * 2**-23 - 1`` for an integer ``k`` uniform in
  ``[0, 2**24)``, which is exact in fp32;
* N(mu, sigma) values are ``mu + sigma * standard_normal()`` drawn in fp64 and
  cast to fp32 by numpy;
* bf16 inputs are such fp32 draws with the low 16 bits dropped (round toward
  zero), stored as their ``uint16`` bit patterns.

The five queue families follow the small-op streams the pages motivate:
"Launch Overhead and Fusion" (section "Fusion": the chain y = relu(a*x + b);
section "Where the time goes": a decoder layer is 10-20 small ops) and
"Kernel Launch and Host-Device Interaction" (section "Why does it exist as a
topic?": a batch-1 decode step is hundreds of ~10 us kernels).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# Opcode names understood by both the oracle and the runtime binding.
EW_UNARY = ("copy", "relu", "exp", "scale")
EW_BINARY = ("add", "mul", "silu_mul")
ROW_OPS = ("row_sum", "row_softmax", "rmsnorm")
ALL_KINDS = (
    "nop", "copy", "gather", "add", "mul", "scale", "relu", "exp",
    "row_sum", "row_softmax", "rmsnorm", "rope", "gemv",
    "attn_score", "attn_av", "silu_mul", "spin", "program",
)

NP_DTYPE = {"f32": np.float32, "bf16": np.uint16, "i32": np.int32, "f16": np.float16}
ELEM_BYTES = {"f32": 4, "bf16": 2, "i32": 4, "f16": 2}


@dataclass(frozen=True)
class Program:
    """The body of an op defined at run time: register instructions
    ``(name, dst, *sources)`` (names as in gpuos_program: mov, add, sub, mul,
    div, min, max, neg, abs, relu, exp, lt, sel), the number of data inputs
    (registers 0..n_inputs-1), the result register and the constants held in
    registers 8..15.  Data only: the oracle and the runtime each give it its
    meaning."""

    insns: Tuple[Tuple, ...]
    n_inputs: int
    result: int
    consts: Tuple[float, ...] = ()


@dataclass(frozen=True)
class Ref:
    """A position inside a named buffer (element offset)."""

    buf: str
    off: int = 0


@dataclass
class Op:
    """One queued small op.

    ``ins`` are the data operands (in[0], in[1]); ``aux`` is the auxiliary
    operand (weight, gain, rotary table or index vector: in[2]).  ``src_len``
    gives the readable length of each data operand (0 = the op's extent).
    ``dims`` holds the integer parameters (GEMV: M, K; attention: H, D, S;
    rotary: heads, head_dim; spin: nanoseconds).  ``deps`` are indices of
    earlier ops in the same workload that this op must wait for, beyond the
    hazards the runtime derives from the byte ranges.  ``view`` (elementwise
    ops only) is (shape, out strides, in0 strides, in1 strides), strides in
    elements from each operand's start.  A ``program`` op reads ``ins``
    (one to three data operands) and runs ``prog``.
    """

    kind: str
    out: Ref
    ins: Tuple[Ref, ...] = ()
    aux: Optional[Ref] = None
    n: int = 0
    dtype: str = "f32"
    rows: int = 0
    row_len: int = 0
    src_len: Tuple[int, int] = (0, 0)
    alpha: float = 0.0
    eps: float = 0.0
    dims: Tuple[int, ...] = ()
    deps: Tuple[int, ...] = ()
    transient: bool = False
    lc: bool = False
    view: Optional[Tuple[Tuple[int, ...], ...]] = None
    prog: Optional[Program] = None


@dataclass
class Workload:
    """A queue of ops plus the initial contents of every buffer it touches."""

    name: str
    buffers: Dict[str, np.ndarray]
    dtypes: Dict[str, str]
    ops: List[Op]
    groups: List[Tuple[int, int]] = field(default_factory=list)
    outputs: List[str] = field(default_factory=list)
    meta: dict = field(default_factory=dict)

    def __post_init__(self):
        if not self.groups:
            self.groups = [(0, len(self.ops))]

    def transient_buffers(self) -> List[str]:
        return sorted({op.out.buf for op in self.ops if op.transient})


# ----------------------------------------------------------------------------
# random draws


def uniform_pm1(rng: np.random.Generator, n: int) -> np.ndarray:
    """U(-1, 1) as exact fp32 values k * 2^-23 - 1."""
    k = rng.integers(0, 1 << 24, size=n, dtype=np.int64)
    return (k.astype(np.float64) * 2.0 ** -23 - 1.0).astype(np.float32)


def normal_f32(rng: np.random.Generator, n: int, mu: float = 0.0, sigma: float = 1.0) -> np.ndarray:
    return (mu + sigma * rng.standard_normal(n)).astype(np.float32)


def f32_to_bf16_trunc(x: np.ndarray) -> np.ndarray:
    """Input preparation only: keep the top 16 bits of each fp32 draw."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def normal_bf16(rng: np.random.Generator, n: int, sigma: float) -> np.ndarray:
    return f32_to_bf16_trunc(normal_f32(rng, n, 0.0, sigma))


# ----------------------------------------------------------------------------
# Queue of 1,000 fp32 elementwise ops on 4,096-element vectors


def gen_elementwise_queue(seed: int = 0, n_ops: int = 1000, n: int = 4096) -> Workload:
    """Random elementwise queue: opcode uniform over add/mul/relu/scale.

    Two seed vectors S0, S1 ~ U(-1, 1); op i reads operands drawn uniformly
    with replacement from {S0, S1, out_0 .. out_{i-1}} (two for add/mul, one
    for relu/scale), scale's alpha ~ U(-1, 1), and writes a fresh out_i.  The
    producers of the operands are listed as explicit dependencies.
    """
    rng = np.random.default_rng(seed)
    bufs = {"S0": uniform_pm1(rng, n), "S1": uniform_pm1(rng, n)}
    dts = {"S0": "f32", "S1": "f32"}
    kinds = ("add", "mul", "relu", "scale")
    ops: List[Op] = []
    names = ["S0", "S1"]
    producer = {"S0": None, "S1": None}
    for i in range(n_ops):
        kind = kinds[int(rng.integers(0, 4))]
        arity = 2 if kind in ("add", "mul") else 1
        srcs = [names[int(rng.integers(0, len(names)))] for _ in range(arity)]
        alpha = float(uniform_pm1(rng, 1)[0]) if kind == "scale" else 0.0
        out = f"o{i}"
        bufs[out] = np.zeros(n, np.float32)
        dts[out] = "f32"
        deps = tuple(sorted({producer[s] for s in srcs if producer[s] is not None}))
        ops.append(Op(kind, Ref(out), tuple(Ref(s) for s in srcs), n=n, alpha=alpha, deps=deps))
        names.append(out)
        producer[out] = i
    return Workload("elementwise_queue", bufs, dts, ops,
                    outputs=[f"o{i}" for i in range(n_ops)],
                    meta={"n": n, "n_ops": n_ops, "bytes": _ew_bytes(ops, dts)})


def _ew_bytes(ops: Sequence[Op], dts: Dict[str, str]) -> int:
    total = 0
    for op in ops:
        eb = ELEM_BYTES[op.dtype]
        total += op.n * eb * (1 + len(op.ins))
    return total


# ----------------------------------------------------------------------------
# Fused chain y = relu(a*x + b)


def gen_fused_chain(seed: int = 0, n: int = 16_777_216) -> Workload:
    """x, a, b ~ N(0, 1) fp32; MUL(a, x) -> t1, ADD(t1, b) -> t2, RELU(t2) -> y.

    t1 and t2 are marked transient so the fusion pass may keep them in
    registers ("Launch Overhead and Fusion", section "Fusion").
    """
    rng = np.random.default_rng(seed)
    bufs = {
        "x": normal_f32(rng, n),
        "a": normal_f32(rng, n),
        "b": normal_f32(rng, n),
        "t1": np.zeros(n, np.float32),
        "t2": np.zeros(n, np.float32),
        "y": np.zeros(n, np.float32),
    }
    dts = {k: "f32" for k in bufs}
    ops = [
        Op("mul", Ref("t1"), (Ref("a"), Ref("x")), n=n, transient=True),
        Op("add", Ref("t2"), (Ref("t1"), Ref("b")), n=n, transient=True, deps=(0,)),
        Op("relu", Ref("y"), (Ref("t2"),), n=n, deps=(1,)),
    ]
    return Workload("fused_chain", bufs, dts, ops, outputs=["y"],
                    meta={"n": n, "fused_bytes": 16 * n, "unfused_bytes": 32 * n})


# relu(a*x + b) as a register program: r3 = r0 * r1; r3 = r3 + r2; r3 = relu(r3)
RELU_AXB = Program((("mul", 3, 0, 1), ("add", 3, 3, 2), ("relu", 3, 3)), n_inputs=3, result=3)


def gen_program_chain(seed: int = 0, n: int = 16_777_216) -> Workload:
    """The fused chain's inputs and result, y = relu(a*x + b), computed by
    one op defined at run time (PROGRAM, inputs a, x, b) instead of the
    built-in MUL, ADD, RELU."""
    base = gen_fused_chain(seed, n)
    bufs = {k: base.buffers[k] for k in ("x", "a", "b", "y")}
    ops = [Op("program", Ref("y"), (Ref("a"), Ref("x"), Ref("b")), n=n, prog=RELU_AXB)]
    return Workload("program_chain", bufs, {k: "f32" for k in bufs}, ops, outputs=["y"],
                    meta={"n": n, "fused_bytes": 16 * n})


# ----------------------------------------------------------------------------
# Batch-1 decode step of a small decoder


def rope_table(positions: Sequence[int], head_dim: int, base: float = 10000.0) -> np.ndarray:
    """Rotary table rows [cos(p*th_i) for i < h/2] + [sin(p*th_i)], th_i = base^(-2i/h).

    Input preparation for the rotary op (computed in fp64, cast to fp32).
    """
    half = head_dim // 2
    inv = base ** (-(2.0 * np.arange(half, dtype=np.float64)) / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


DECODE_OPS_PER_LAYER = 15


def gen_decode(seed: int = 0, layers: int = 24, hidden: int = 896, heads: int = 14,
               head_dim: int = 64, ffn: int = 4864, kv_len: int = 512, tokens: int = 64,
               eps: float = 1e-6, weight_std: float = 0.02, distinct: bool = False) -> Workload:
    """Synthetic batch-1 decode of a decoder with random N(0, 0.02) bf16 weights.

    Per layer, 15 ops: RMSNORM, GEMV(qkv), ROPE(q), ROPE(k -> K cache slot),
    COPY(v -> V cache slot), ATTN_SCORE, ROW_SOFTMAX, ATTN_AV, GEMV(o), ADD,
    RMSNORM, GEMV(gate|up), SILU_MUL, GEMV(down), ADD.  Token t sits at
    position kv_len + t and writes cache slot t mod kv_len; attention covers all
    kv_len slots (a sliding window over a random N(0, 1) cache).  The hidden
    state after the last layer of token t is the input of token t + 1.  Each
    token's ops form one submission group (flush per token).

    With ``distinct`` every activation of every (token, layer) gets its own
    buffer and the residual adds write a new hidden-state buffer, so each
    element is written at most once (verification mode: every intermediate
    survives to the end and each op can be re-checked on its own inputs).
    """
    assert hidden == heads * head_dim
    rng = np.random.default_rng(seed)
    H, Dh, D, F, S = heads, head_dim, hidden, ffn, kv_len
    bufs: Dict[str, np.ndarray] = {}
    dts: Dict[str, str] = {}

    def add(name, arr, dt):
        bufs[name] = arr
        dts[name] = dt

    for l in range(layers):
        add(f"Wqkv{l}", normal_bf16(rng, 3 * D * D, weight_std), "bf16")
        add(f"Wo{l}", normal_bf16(rng, D * D, weight_std), "bf16")
        add(f"Wgu{l}", normal_bf16(rng, 2 * F * D, weight_std), "bf16")
        add(f"Wdown{l}", normal_bf16(rng, D * F, weight_std), "bf16")
        add(f"gin{l}", normal_bf16(rng, D, weight_std), "bf16")
        add(f"gpost{l}", normal_bf16(rng, D, weight_std), "bf16")
        add(f"K{l}", normal_bf16(rng, S * D, 1.0), "bf16")
        add(f"V{l}", normal_bf16(rng, S * D, 1.0), "bf16")
    add("x", normal_bf16(rng, D, 1.0), "bf16")
    for name, cnt, dt in (("h", D, "bf16"), ("qkv", 3 * D, "bf16"), ("q", D, "bf16"),
                          ("scores", H * S, "f32"), ("probs", H * S, "f32"),
                          ("attn", D, "bf16"), ("o", D, "bf16"), ("gu", 2 * F, "bf16"),
                          ("act", F, "bf16"), ("down", D, "bf16")):
        add(name, np.zeros(cnt, NP_DTYPE[dt]), dt)
    add("rope", rope_table([S + t for t in range(tokens)], Dh).reshape(-1), "f32")

    eps32 = float(np.float32(eps))
    ops: List[Op] = []
    groups = []
    sizes = {"h": (D, "bf16"), "qkv": (3 * D, "bf16"), "q": (D, "bf16"),
             "scores": (H * S, "f32"), "probs": (H * S, "f32"), "attn": (D, "bf16"),
             "o": (D, "bf16"), "gu": (2 * F, "bf16"), "act": (F, "bf16"), "down": (D, "bf16"),
             "x": (D, "bf16")}
    cur_x = "x"
    for t in range(tokens):
        g0 = len(ops)
        slot = t % S
        tab = Ref("rope", t * Dh)
        for l in range(layers):
            if distinct:
                def nm(base, tag=""):
                    name = f"{base}{tag}.{t}.{l}"
                    cnt, dt = sizes[base]
                    if name not in bufs:
                        add(name, np.zeros(cnt, NP_DTYPE[dt]), dt)
                    return name
                h1, qkv, q, sc, pr = nm("h", "a"), nm("qkv"), nm("q"), nm("scores"), nm("probs")
                at, o, h2, gu, act, dn = nm("attn"), nm("o"), nm("h", "b"), nm("gu"), nm("act"), nm("down")
                x_in, x_mid, x_out = cur_x, nm("x", "a"), nm("x", "b")
            else:
                h1 = h2 = "h"
                qkv, q, sc, pr, at, o, gu, act, dn = ("qkv", "q", "scores", "probs", "attn", "o",
                                                      "gu", "act", "down")
                x_in = x_mid = x_out = "x"
            ops += [
                Op("rmsnorm", Ref(h1), (Ref(x_in),), Ref(f"gin{l}"), n=D, dtype="bf16",
                   rows=1, row_len=D, eps=eps32),
                Op("gemv", Ref(qkv), (Ref(h1),), Ref(f"Wqkv{l}"), n=3 * D, dtype="bf16",
                   dims=(3 * D, D)),
                Op("rope", Ref(q), (Ref(qkv, 0),), tab, n=D, dtype="bf16",
                   rows=H, row_len=Dh, dims=(H, Dh)),
                Op("rope", Ref(f"K{l}", slot * D), (Ref(qkv, D),), tab, n=D, dtype="bf16",
                   rows=H, row_len=Dh, dims=(H, Dh)),
                Op("copy", Ref(f"V{l}", slot * D), (Ref(qkv, 2 * D),), n=D, dtype="bf16"),
                Op("attn_score", Ref(sc), (Ref(q),), Ref(f"K{l}"), n=H * S,
                   dtype="bf16", alpha=1.0 / math.sqrt(Dh), dims=(H, Dh, S)),
                Op("row_softmax", Ref(pr), (Ref(sc),), n=H * S, dtype="f32",
                   rows=H, row_len=S),
                Op("attn_av", Ref(at), (Ref(pr),), Ref(f"V{l}"), n=D, dtype="bf16",
                   dims=(H, Dh, S)),
                Op("gemv", Ref(o), (Ref(at),), Ref(f"Wo{l}"), n=D, dtype="bf16",
                   dims=(D, D)),
                Op("add", Ref(x_mid), (Ref(x_in), Ref(o)), n=D, dtype="bf16"),
                Op("rmsnorm", Ref(h2), (Ref(x_mid),), Ref(f"gpost{l}"), n=D, dtype="bf16",
                   rows=1, row_len=D, eps=eps32),
                Op("gemv", Ref(gu), (Ref(h2),), Ref(f"Wgu{l}"), n=2 * F, dtype="bf16",
                   dims=(2 * F, D)),
                Op("silu_mul", Ref(act), (Ref(gu, 0), Ref(gu, F)), n=F, dtype="bf16"),
                Op("gemv", Ref(dn), (Ref(act),), Ref(f"Wdown{l}"), n=D, dtype="bf16",
                   dims=(D, F)),
                Op("add", Ref(x_out), (Ref(x_mid), Ref(dn)), n=D, dtype="bf16"),
            ]
            cur_x = x_out
        groups.append((g0, len(ops)))
    weight_bytes = 2 * layers * (3 * D * D + D * D + 2 * F * D + D * F + 2 * D)
    kv_bytes = 2 * layers * 2 * S * D
    outs = [cur_x] + [f"K{l}" for l in range(layers)] + [f"V{l}" for l in range(layers)]
    if distinct:
        outs = sorted({op.out.buf for op in ops})
    return Workload("decode", bufs, dts, ops, groups=groups, outputs=outs,
                    meta={"layers": layers, "tokens": tokens, "hidden": D, "heads": H,
                          "head_dim": Dh, "ffn": F, "kv_len": S,
                          "weight_bytes": weight_bytes, "kv_bytes": kv_bytes,
                          "ops_per_token": layers * DECODE_OPS_PER_LAYER, "final_x": cur_x})


# ----------------------------------------------------------------------------
# Dynamic-shape random-DAG stream


def _log_uniform_int(rng, lo: int, hi: int) -> int:
    v = int(math.floor(math.exp(rng.uniform(math.log(lo), math.log(hi + 1)))))
    return min(max(v, lo), hi)


def gen_dynamic_dag(seed: int = 0, n_ops: int = 100_000, n_min: int = 256,
                    n_max: int = 1 << 20, pool: int = 16, pool_len: int = 1 << 20,
                    ring: int = 64, distinct_outputs: bool = False,
                    row_min: int = 128, row_max: int = 4096, window: int = 8,
                    group: int = 0) -> Workload:
    """Stream of ops with log-uniform sizes and random DAG dependencies.

    Opcode uniform over add/mul/relu/exp/row_sum/row_softmax; n log-uniform in
    [n_min, n_max]; row ops draw a row length L log-uniform in [row_min,
    row_max] and use rows = max(1, n // L), n = rows * L.  Each op depends on
    k ~ U{0, 1, 2} distinct ops among the previous ``window``; the first
    min(k, arity) of them supply its inputs in order, the rest are
    ordering-only dependencies, and missing inputs come from a pool of U(-1, 1)
    vectors.  A source shorter than the op's extent is read cyclically.
    Outputs go to a ring of ``ring`` slots (write-after-read reuse), or to one
    buffer per op when ``distinct_outputs`` is set.  ``group`` > 0 splits the
    stream into submission groups of that many ops.
    """
    rng = np.random.default_rng(seed)
    kinds = ("add", "mul", "relu", "exp", "row_sum", "row_softmax")
    bufs: Dict[str, np.ndarray] = {}
    dts: Dict[str, str] = {}
    for p in range(pool):
        bufs[f"p{p}"] = uniform_pm1(rng, pool_len)
        dts[f"p{p}"] = "f32"
    if not distinct_outputs:
        for r in range(ring):
            bufs[f"r{r}"] = np.zeros(n_max, np.float32)
            dts[f"r{r}"] = "f32"
    ops: List[Op] = []
    out_len: List[int] = []
    for i in range(n_ops):
        kind = kinds[int(rng.integers(0, len(kinds)))]
        n = _log_uniform_int(rng, n_min, n_max)
        rows = row_len = 0
        if kind in ("row_sum", "row_softmax"):
            row_len = _log_uniform_int(rng, row_min, row_max)
            rows = max(1, n // row_len)
            n = rows * row_len
        arity = 2 if kind in ("add", "mul") else 1
        k = min(int(rng.integers(0, 3)), i)
        lo = max(0, i - window)
        deps = [int(d) for d in rng.choice(np.arange(lo, i), size=k, replace=False)] if k else []
        ins: List[Ref] = []
        src: List[int] = []
        for a in range(arity):
            if a < len(deps):
                d = deps[a]
                ins.append(ops[d].out)
                src.append(out_len[d])
            else:
                p = int(rng.integers(0, pool))
                ins.append(Ref(f"p{p}"))
                src.append(pool_len)
        olen = rows if kind == "row_sum" else n
        if distinct_outputs:
            name = f"o{i}"
            bufs[name] = np.zeros(olen, np.float32)
            dts[name] = "f32"
        else:
            name = f"r{i % ring}"
        src_len = tuple(src + [0] * (2 - len(src)))
        ops.append(Op(kind, Ref(name), tuple(ins), n=n, rows=rows, row_len=row_len,
                      src_len=src_len, deps=tuple(sorted(deps))))
        out_len.append(olen)
    groups = [(s, min(s + group, n_ops)) for s in range(0, n_ops, group)] if group else []
    algo = 0
    for op, ol in zip(ops, out_len):
        algo += 4 * (op.n * len(op.ins) + ol)
    outs = [f"o{i}" for i in range(n_ops)] if distinct_outputs else [f"r{r}" for r in range(ring)]
    return Workload("dynamic_dag", bufs, dts, ops, groups=groups, outputs=outs,
                    meta={"n_ops": n_ops, "bytes": algo, "out_len": out_len})


# ----------------------------------------------------------------------------
# Two-priority mixed queue


def gen_priority_mix(seed: int = 0, rounds: int = 200, lc_per_round: int = 10,
                     lc_n: int = 4096, be_n: int = 67_108_864, eps: float = 1e-6) -> Workload:
    """Latency-critical bf16[4096] ops interleaved 10:1 with best-effort fp32 ops.

    LC opcode uniform over add/mul/relu/scale/rmsnorm (one row of lc_n, gain ~
    U(-1, 1)) reading 8 fixed U(-1, 1) vectors and writing one output buffer
    per LC op; BE opcode uniform over add/mul/relu/scale on fp32[be_n] operands
    drawn from 3 U(-1, 1) buffers, outputs alternating between 2 buffers.  The
    op order is round by round: one BE op, then lc_per_round LC ops.
    """
    rng = np.random.default_rng(seed)
    bufs: Dict[str, np.ndarray] = {}
    dts: Dict[str, str] = {}
    for j in range(8):
        bufs[f"L{j}"] = f32_to_bf16_trunc(uniform_pm1(rng, lc_n))
        dts[f"L{j}"] = "bf16"
    bufs["Lg"] = f32_to_bf16_trunc(uniform_pm1(rng, lc_n))
    dts["Lg"] = "bf16"
    for j in range(3):
        bufs[f"B{j}"] = uniform_pm1(rng, be_n)
        dts[f"B{j}"] = "f32"
    for j in range(2):
        bufs[f"Bo{j}"] = np.zeros(be_n, np.float32)
        dts[f"Bo{j}"] = "f32"
    eps32 = float(np.float32(eps))
    ops: List[Op] = []
    lc_kinds = ("add", "mul", "relu", "scale", "rmsnorm")
    be_kinds = ("add", "mul", "relu", "scale")
    lc_index = 0
    for r in range(rounds):
        kind = be_kinds[int(rng.integers(0, 4))]
        ar = 2 if kind in ("add", "mul") else 1
        ins = tuple(Ref(f"B{int(rng.integers(0, 3))}") for _ in range(ar))
        alpha = float(uniform_pm1(rng, 1)[0]) if kind == "scale" else 0.0
        ops.append(Op(kind, Ref(f"Bo{r % 2}"), ins, n=be_n, alpha=alpha))
        for _ in range(lc_per_round):
            kind = lc_kinds[int(rng.integers(0, 5))]
            name = f"lo{lc_index}"
            lc_index += 1
            bufs[name] = np.zeros(lc_n, np.uint16)
            dts[name] = "bf16"
            if kind == "rmsnorm":
                ops.append(Op("rmsnorm", Ref(name), (Ref(f"L{int(rng.integers(0, 8))}"),), Ref("Lg"),
                              n=lc_n, dtype="bf16", rows=1, row_len=lc_n, eps=eps32, lc=True))
            else:
                ar = 2 if kind in ("add", "mul") else 1
                ins = tuple(Ref(f"L{int(rng.integers(0, 8))}") for _ in range(ar))
                alpha = float(uniform_pm1(rng, 1)[0]) if kind == "scale" else 0.0
                ops.append(Op(kind, Ref(name), ins, n=lc_n, dtype="bf16", alpha=alpha, lc=True))
    return Workload("priority_mix", bufs, dts, ops,
                    outputs=["Bo0", "Bo1"] + [f"lo{i}" for i in range(lc_index)],
                    meta={"rounds": rounds, "lc_per_round": lc_per_round})
