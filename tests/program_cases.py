"""Program cases shared by the program tests: input values with IEEE
special cases, every instruction alone, chains of them, and workloads of
program ops over those inputs."""

import numpy as np

import oracle
from persistent_fusion_amd import gpuos, workloads
from persistent_fusion_amd.workloads import Op, Program, Ref, Workload


def specials(rng, n):
    """Random values with NaN, +-0, +-inf, subnormals, ties and huge/tiny
    magnitudes spread through them."""
    v = (rng.standard_normal(n) * np.exp2(rng.integers(-20, 20, n))).astype(np.float32)
    sp = np.array([np.nan, 0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45, 1.17e-38, 3.0e38, -3.0e38,
                   1.0, -1.0, 0.5, 2.0], np.float32)
    idx = rng.choice(n, size=min(n, 4 * len(sp)), replace=False)
    v[idx] = np.resize(sp, idx.size)
    return v


# every instruction once, each in its own one-instruction program, plus
# programs that chain them
SINGLE = [(name, 3) + tuple(range(gpuos.POP_ARITY[name])) for name in gpuos.POPS]
CHAINS = [
    Program((("mul", 3, 0, 1), ("add", 3, 3, 2), ("relu", 3, 3)), 3, 3),
    Program((("sub", 3, 0, 1), ("div", 4, 3, 2), ("max", 5, 4, 8), ("min", 5, 5, 9), ("abs", 6, 5),
             ("neg", 6, 6), ("lt", 7, 6, 0), ("sel", 3, 7, 4, 5)), 3, 3, consts=(-4.0, 4.0)),
    Program((("neg", 3, 0), ("exp", 3, 3), ("add", 3, 3, 8), ("div", 3, 0, 3), ("mul", 3, 3, 1)),
            2, 3, consts=(1.0,)),                                   # x * sigmoid(x) * u
    Program((("add", 4, 0, 5), ("mul", 4, 4, 9), ("mov", 1, 4)), 1, 1, consts=(0.0, -0.75)),  # r5 = +0
]


def program_workload(progs, n, dtype, seed, misalign=False, in_place=False):
    rng = np.random.default_rng(seed)
    npdt = workloads.NP_DTYPE[dtype]
    off = 1 if misalign else 0
    bufs, dts, ops = {}, {}, []
    for k, prog in enumerate(progs):
        ins = []
        for j in range(prog.n_inputs):
            name = f"p{k}_{j}"
            v = specials(rng, n + off)
            if dtype == "bf16":
                v = oracle.f32_to_bf16(v)
            bufs[name] = v.astype(npdt) if dtype != "bf16" else v
            dts[name] = dtype
            ins.append(Ref(name, off))
        out = ins[0] if in_place else Ref(f"y{k}", off)
        if not in_place:
            bufs[f"y{k}"] = np.zeros(n + off, npdt)
            dts[f"y{k}"] = dtype
        ops.append(Op("program", out, tuple(ins), n=n, dtype=dtype, prog=prog))
    outs = sorted({op.out.buf for op in ops})
    return Workload("programs", bufs, dts, ops, outputs=outs)
