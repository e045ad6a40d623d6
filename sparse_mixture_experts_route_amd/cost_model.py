"""Per-phase analytic cost model of the MoE layer forward on MI355X.

The MOSAIC summary ("Compute-Optimal Is Not Cluster-Optimal", gist.science,
method item 2, the operator-level performance model) predicts the MFU of a
layout from per-operator costs (grouped GEMMs, dispatch latency of small
batches among them) and judges the model by its mean absolute percentage
error (MAPE) on measured runs.
This module does the same for the four phases of this layer as this library
runs them on one GPU. Every phase time is linear in a few terms taken from
the kernels' own work and schedule, so the constants are a least-squares fit:

  route     a0 + (a1 + a2 * E64 / 64) * K steps of 64 in the busiest CU's
            chain of router blocks + a3 * thousands of partial logits a
            finalize wave adds per token (splits x E; small batches split
            d_model) + a4 * M selections (a block scores 64 tokens, or 32
            where 64-token blocks would leave CUs idle, against the E64
            experts padded to 64; most layers give every CU at most one
            round of such blocks, so the serial chain, not HBM, sets the
            time)
  permute   b0 + b1 * [one-workgroup form, T <= 1024] + b2 * [separate
            scan launch, more than 64 blocks of 256 tokens] + b3 * M
            selections (index arrays only: the token rows reach the first
            GEMM through perm)
  ffn       f0 * launches (each GEMM, and its fixup unless split tiles are
            completed inside the launch or K is too short to split) + f1 * K
            steps of 64 run by the busiest persistent block of a matrix-core
            tile + f2 * tiles that block runs + f3 * MB of split-tile partial
            sums written and read back + f4 * K steps of the busiest block of
            the 32-row weight-streaming tile + f5 * MB of weight slabs that
            tile streams (the experts with rows). f0 comes out near zero: the
            step count charges in full the first and last steps of a tile,
            which the pipeline overlaps with its neighbours
  combine   c0 + c1 * MB read and written (plain accesses) + c2 * MB read
            and written (non-temporal, y_perm of 128 MB or more) + c3 *
            thousands of elements one token's wave reads (k rows of d_model:
            the latency chain of small batches)

The terms replay the launcher's decisions: the router split, the permute
form, the GEMM tile per problem, tiles per expert group dealt to 8 XCDs x
(CUs / 8) persistent blocks, whole rounds first and a leftover round of long
tiles split over the blocks by K steps.

The model covers the bf16 layer. `measure()` times the phases on the GPU
through the library's stage entry points (the whole-layer path's own calls);
`fit()`, `predict()` and `calibrated()` (constants from the committed MI355X
samples, cost_samples_mi355x.json, written by `main()`) run on the host only.
"""

from __future__ import annotations

import json
import math
import os
from dataclasses import asdict, dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

PHASES = ("route", "permute", "ffn", "combine")
CUS = 256
TILE = 256
SPLIT_MIN_STEPS = 24


@dataclass
class Sample:
    """One measured layer shape: sizes, per-expert selection counts, phase times (us)."""
    T: int
    d_model: int
    E: int
    k: int
    d_expert: int
    counts: List[int]
    phases_us: Dict[str, float] = field(default_factory=dict)

    @property
    def step_us(self) -> float:
        return sum(self.phases_us[p] for p in PHASES)


def balanced_counts(T: int, E: int, k: int) -> List[int]:
    R = T * k
    return [R // E + (1 if e < R % E else 0) for e in range(E)]


# GEMM block tiles (name, BM, BN, BK, blocks per CU, matrix-core efficiency
# relative to the 8-wave 256 x 256 tile; 0 = never picked on its own), as the
# library's grouped GEMM launcher knows them.
SHAPES = [
    ("256x256", 256, 256, 64, 1, 0.0), ("256x256k32", 256, 256, 32, 1, 0.0),
    ("256x128", 256, 128, 32, 2, 0.8), ("128x128", 128, 128, 64, 2, 0.75),
    ("128x128k32", 128, 128, 32, 2, 0.0), ("256x256w8", 256, 256, 64, 1, 1.0),
    ("256x256w8k32", 256, 256, 32, 1, 0.0),
    ("32x256", 32, 256, 64, 1, 0.0),  # weight streaming: picked by row count, not by score
]
DECODE_TILE = 7


def _split(rem: int, nb: int, nk: int, max_rem: Optional[int] = None) -> bool:
    max_rem = nb // 3 if max_rem is None else max_rem
    return 0 < rem <= max_rem and nk * (nb - rem) >= SPLIT_MIN_STEPS * nb


def pick_tile(R: int, K: int, N: int, E: int) -> int:
    """The launcher's tile choice: the 32-row streaming tile for at most ~40
    rows per expert, else the best product of tile efficiency, round
    occupancy and row-padding efficiency."""
    if R <= 40 * E and K % 64 == 0:
        return DECODE_TILE
    best, best_score = 5, -1.0
    for c, (_, bm, bn, bk, occ, eff) in enumerate(SHAPES):
        if eff <= 0.0 or K % bk:
            continue
        m_tiles = R / bm + 0.5 * E
        rounds = m_tiles * math.ceil(N / bn) / (CUS * occ)
        whole = float(int(rounds))
        frac = rounds - whole
        if rounds < 1.0:
            round_eff = rounds
        elif frac * 3.0 <= 1.0 and (K // bk) * (1.0 - frac) >= SPLIT_MIN_STEPS:
            round_eff = rounds / (rounds + 0.1)
        else:
            round_eff = rounds / (whole + 1.0 if frac > 0.0 else whole)
        score = eff * round_eff * R / (m_tiles * bm)
        if score > best_score:
            best, best_score = c, score
    return best


def gemm_plan(counts: Sequence[int], K: int, N: int, E: int, gelu: bool) -> Dict[str, int]:
    """One grouped GEMM launch as the library plans it (the fields of
    moe_gemm_plan_t): tile, persistent grid (8 XCDs x blocks), K steps, the
    split rule, in-launch completion of split tiles, and the tile list of
    these per-expert counts dealt to the XCDs in contiguous eighths."""
    R = sum(counts)
    shape = pick_tile(R, K, N, E)
    _, bm, bn, bk, occ, _ = SHAPES[shape]
    stream = shape == DECODE_TILE
    n_t = math.ceil(N / bn)
    tiles = sum(math.ceil(c / bm) for c in counts) * n_t
    tiles_ub = ((R + E * (bm - 1)) // bm) * n_t
    grid = CUS * occ if stream else max(8, min(math.ceil(tiles_ub / 8) * 8, CUS * occ))
    nb = grid // 8
    nk = K // bk
    max_rem = nb - 1 if stream else nb // 3
    xcd = [tiles * (x + 1) // 8 - tiles * x // 8 for x in range(8)]
    full, rem = divmod(max(xcd), nb)
    return {"tile": shape, "bm": bm, "bn": bn, "bk": bk, "grid": grid, "k_steps": nk, "max_split": max_rem,
            "min_steps": SPLIT_MIN_STEPS, "split_in_launch": int(stream and gelu and 2 * R >= E),
            "tiles": tiles, "xcd_rounds": full, "xcd_leftover": rem,
            "xcd_split": int(_split(rem, nb, nk, max_rem)),
            "split_xcds": sum(int(_split(t % nb, nb, nk, max_rem)) for t in xcd)}


def _gemm_terms(counts: Sequence[int], K: int, N: int, E: int, gelu: bool) -> Dict[str, float]:
    """Work of the busiest persistent block of one grouped-GEMM launch: K
    steps of 64 in units of the 8-wave 256 x 256 tile (scaled by the tile's
    MAC count, blocks sharing a CU and matrix-core efficiency), tiles begun,
    split partial sums moved, K steps of the weight-streaming tile, and the
    fixup launch (absent when split tiles are completed inside the launch)."""
    g = gemm_plan(counts, K, N, E, gelu)
    _, bm, bn, bk, occ, eff = SHAPES[g["tile"]]
    stream = g["tile"] == DECODE_TILE
    nb, nk, full, rem = g["grid"] // 8, g["k_steps"], g["xcd_rounds"], g["xcd_leftover"]
    if g["xcd_split"]:
        steps = full * nk + math.ceil(rem * nk / nb)
        n_tiles = full + 1
        partial_mb = 2 * 8 * nb * bm * bn * 4 / 1e6  # every block writes a share, the fixup reads it
    else:
        n_tiles = full + (1 if rem else 0)
        steps = n_tiles * nk
        partial_mb = 0.0
    fixup = 0.0 if g["split_in_launch"] or not (nk >= SPLIT_MIN_STEPS and g["max_split"] > 0) else 1.0
    if stream:
        # the weight slabs of the experts with rows, streamed once from HBM
        weight_mb = sum(1 for c in counts if c > 0) * K * N * 2 / 1e6
        return {"steps": 0.0, "tiles": n_tiles, "partial_mb": partial_mb, "stream_steps": steps, "fixup": fixup,
                "stream_mb": weight_mb}
    scale = (bm * bn * bk * occ) / (256 * 256 * 64) / eff
    return {"steps": steps * scale, "tiles": n_tiles * occ, "partial_mb": partial_mb, "stream_steps": 0.0,
            "fixup": fixup, "stream_mb": 0.0}


def route_rt(T: int, E: int) -> int:
    """Tokens per router block: 32 where 64-token blocks would fill a quarter
    to all of the CUs (too many to split over d_model) and E <= 128, else 64."""
    b64 = math.ceil(T / 64)
    return 32 if E <= 128 and b64 * 4 > CUS and b64 < CUS else 64


def route_splits(T: int, d: int, E: int) -> int:
    """The router's split over d_model: only when the router blocks fill at
    most a quarter of the CUs; about two blocks per CU, at least four K steps
    per split, at most 64 KB of partial logits per token."""
    blocks = math.ceil(T / route_rt(T, E))
    if E % 8 or blocks * 4 > CUS:
        return 1
    ns = min(math.ceil(2 * CUS / blocks), (d // 64) // 4, 65536 // (E * 4))
    return max(ns, 1)


def _route_blocks_per_cu(ep: int, rt: int = 64) -> int:
    """Router blocks one CU holds at once: its LDS ring of rt x 64 token
    pieces and 64 x E64 weight pieces (4 stages up to 128 experts, else 3),
    or the float32 logits of the block when larger, out of 160 KB."""
    stages = 4 if ep <= 128 else 3
    smem = max(stages * (rt * 64 * 2 + 64 * ep * 2), rt * (ep + 1) * 4)
    return max(1, 160 * 1024 // smem)


COMBINE_STREAM_BYTES = 128 << 20  # y_perm size from which the combine streams (non-temporal accesses)
FUSED_ROUTE_T = 16  # tokens up to which moe_forward's permute workgroup completes a split router


def plan(T: int, d_model: int, E: int, k: int, d_expert: int, counts: Optional[Sequence[int]] = None) -> Dict:
    """The bf16 layer's launch decisions as this model restates them, in the
    form of the library's moe_plan (include/moe.h): router split and block,
    permute form, combine mode and both grouped GEMMs (their tile lists only
    with counts). The tests hold the two equal."""
    R = T * k
    ns = route_splits(T, d_model, E)
    small = T <= 1024 and k <= 8
    out = {"route_splits": ns, "route_tokens_per_block": route_rt(T, E),
           "route_fused_permute": int(ns > 1 and T <= FUSED_ROUTE_T and k <= 8 and ns * T * E * 4 <= 256 * 1024),
           "permute_form": 0 if small else (1 if math.ceil(T / 256) <= 64 else 2),
           "gather_in_gemm": int(T * d_model * 2 < 2 ** 31 - 1),
           "combine_streaming": int(R * d_model * 2 >= COMBINE_STREAM_BYTES)}
    c = list(counts) if counts is not None else balanced_counts(T, E, k)
    gemms = [gemm_plan(c, d_model, d_expert, E, True), gemm_plan(c, d_expert, d_model, E, False)]
    if counts is None:
        for g in gemms:
            for key in ("tiles", "xcd_rounds", "xcd_leftover", "xcd_split", "split_xcds"):
                g[key] = -1
    out["gemm"] = gemms
    out["forward_one_launch"] = 0  # the one-launch layer is float32 only
    return out


def features(s: Sample) -> Dict[str, np.ndarray]:
    """Design rows of the four linear phase models (bf16 layer)."""
    T, d, E, k, de = s.T, s.d_model, s.E, s.k, s.d_expert
    R = T * k
    es = 2
    ep = math.ceil(E / 64) * 64
    pl = plan(T, d, E, k, de)
    ns, rt = pl["route_splits"], pl["route_tokens_per_block"]
    rounds = math.ceil(math.ceil(T / rt) * ns / (CUS * _route_blocks_per_cu(ep, rt)))
    chain = rounds * math.ceil(d / 64 / ns)
    small = 1.0 if pl["permute_form"] == 0 else 0.0
    scan_launch = 1.0 if pl["permute_form"] == 2 else 0.0
    mb = (R * d * es + T * d * es) / 1e6
    stream = pl["combine_streaming"]
    g1 = _gemm_terms(s.counts, d, de, E, True)
    g2 = _gemm_terms(s.counts, de, d, E, False)
    return {
        "route": np.array([1.0, chain, chain * ep / 64, (ns * E / 1e3) if ns > 1 else 0.0, R / 1e6]),
        "permute": np.array([1.0, small, scan_launch, R / 1e6]),
        "ffn": np.array([2.0 + g1["fixup"] + g2["fixup"], g1["steps"] + g2["steps"], g1["tiles"] + g2["tiles"],
                         g1["partial_mb"] + g2["partial_mb"], g1["stream_steps"] + g2["stream_steps"],
                         g1["stream_mb"] + g2["stream_mb"]]),
        "combine": np.array([1.0, 0.0 if stream else mb, mb if stream else 0.0, k * d / 1e3]),
    }


@dataclass
class CostModel:
    coef: Dict[str, List[float]]

    def predict(self, T: int, d_model: int, E: int, k: int, d_expert: int,
                counts: Sequence[int]) -> Dict[str, float]:
        """Predicted phase times (us) and their sum ("step") for the per-expert
        selection counts of the routing at hand (e.g. moe_permute's counts;
        balanced_counts() only for a perfectly balanced router: a real
        router's imbalance adds tiles)."""
        if counts is None or len(counts) != E or sum(counts) != T * k:
            raise ValueError("predict needs the E per-expert selection counts of the routing (summing to T * k)")
        s = Sample(T, d_model, E, k, d_expert, [int(c) for c in counts])
        f = features(s)
        out = {p: float(f[p] @ np.asarray(self.coef[p])) for p in PHASES}
        out["step"] = sum(out[p] for p in PHASES)
        return out

    def to_json(self) -> str:
        return json.dumps({"coef": self.coef}, indent=1)

    @staticmethod
    def from_json(text: str) -> "CostModel":
        return CostModel(coef=json.loads(text)["coef"])


def fit(samples: Sequence[Sample]) -> CostModel:
    """Least-squares constants per phase, weighted by 1/time so that the fit
    minimises relative rather than absolute error."""
    coef = {}
    for p in PHASES:
        X = np.stack([features(s)[p] for s in samples])
        y = np.array([s.phases_us[p] for s in samples])
        w = 1.0 / y
        c, *_ = np.linalg.lstsq(X * w[:, None], y * w, rcond=None)
        coef[p] = [float(v) for v in c]
    return CostModel(coef)


def mfu(T: int, d_model: int, k: int, d_expert: int, step_us: float, peak_flops: float = 2.5e15) -> float:
    """Model-FLOPs utilisation of one layer step: the expert GEMMs' 4 T k d d_e
    flops over the step time, against the bf16 dense matrix-core peak."""
    return 4.0 * T * k * d_model * d_expert / (step_us * 1e-6) / peak_flops


def mape(model: CostModel, samples: Sequence[Sample]) -> Dict[str, float]:
    """Mean absolute percentage error per phase, for the whole step, and of
    the step's MFU (the performance model's own yardstick)."""
    errs = {p: [] for p in PHASES + ("step", "mfu")}
    for s in samples:
        pr = model.predict(s.T, s.d_model, s.E, s.k, s.d_expert, s.counts)
        for p in PHASES:
            errs[p].append(abs(pr[p] - s.phases_us[p]) / s.phases_us[p])
        errs["step"].append(abs(pr["step"] - s.step_us) / s.step_us)
        m_meas = mfu(s.T, s.d_model, s.k, s.d_expert, s.step_us)
        m_pred = mfu(s.T, s.d_model, s.k, s.d_expert, pr["step"])
        errs["mfu"].append(abs(m_pred - m_meas) / m_meas)
    return {p: 100.0 * float(np.mean(v)) for p, v in errs.items()}


SAMPLES_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "cost_samples_mi355x.json")


def calibrated() -> CostModel:
    """The model fitted on every committed MI355X sample."""
    return fit(load_samples(SAMPLES_FILE))


def load_samples(path: str) -> List[Sample]:
    return [Sample(**r) for r in json.load(open(path))]


def save_samples(samples: Sequence[Sample], path: str) -> None:
    json.dump([asdict(s) for s in samples], open(path, "w"), indent=1)


def measure(T: int, d_model: int, E: int, k: int, d_expert: int, steps: int = 10, warmup: int = 30,
            seed: int = 0) -> Sample:
    """Phase times of one bf16 shape on the current GPU (random inputs of the
    workloads' distributions: x ~ N(0,1), router std 0.02, fan-in scaled
    expert weights), through the stage calls the whole-layer path makes."""
    import torch

    from . import _lib as lib

    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(seed)

    def randn(shape, std):
        return (torch.randn(shape, generator=g, device=dev) * std).to(torch.bfloat16)

    x = randn((T, d_model), 1.0)
    wr = randn((d_model, E), 0.02)
    W1 = randn((E, d_model, d_expert), d_model ** -0.5)
    W2 = randn((E, d_expert, d_model), d_expert ** -0.5)
    p = lib.make_problem(T, d_model, E, k, d_expert, torch.bfloat16)
    R = T * k
    i32 = dict(dtype=torch.int32, device=dev)
    idx, gate = torch.empty((T, k), **i32), torch.empty((T, k), dtype=torch.float32, device=dev)
    counts, offsets = torch.empty(E, **i32), torch.empty(E + 1, **i32)
    perm, inv = torch.empty(R, **i32), torch.empty(R, **i32)
    y_perm = torch.empty((R, d_model), dtype=torch.bfloat16, device=dev)
    y = torch.empty((T, d_model), dtype=torch.bfloat16, device=dev)
    ws_r = torch.empty(lib.moe_workspace_size(p, lib.MOE_STAGE_ROUTE), dtype=torch.uint8, device=dev)
    ws_p = torch.empty(lib.moe_workspace_size(p, lib.MOE_STAGE_PERMUTE), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(lib.moe_workspace_size(p, lib.MOE_STAGE_GROUPED_FFN), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        lib.moe_route_ws(p, x, wr, None, None, idx, gate, ws_r)
        if ev:
            ev[1].record(stream)
        lib.moe_permute_index(p, idx, counts, offsets, perm, inv, ws_p)
        if ev:
            ev[2].record(stream)
        lib.moe_grouped_ffn_gather(p, x, perm, offsets, W1, W2, y_perm, ws_f)
        if ev:
            ev[3].record(stream)
        lib.moe_combine(p, y_perm, inv, gate, y)
        if ev:
            ev[4].record(stream)

    for _ in range(warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    ph = {n: 1000.0 * sorted(e[i].elapsed_time(e[i + 1]) for e in evs)[steps // 2] for i, n in enumerate(PHASES)}
    return Sample(T, d_model, E, k, d_expert, [int(c) for c in counts.cpu()], ph)


# Shapes of the committed calibration data: a fitting set and a held-out set.
FIT_SHAPES = [
    (4096, 2048, 8, 2, 8192), (8192, 2048, 64, 8, 1024), (16384, 2048, 64, 8, 1024),
    (2048, 1024, 16, 2, 4096), (8192, 4096, 32, 4, 2048), (4096, 1024, 64, 8, 512),
    (16384, 1024, 8, 1, 4096), (1024, 2048, 8, 2, 8192), (8192, 2048, 128, 8, 768),
    (32768, 1024, 32, 2, 1024), (4096, 4096, 8, 2, 4096), (12288, 2048, 16, 4, 2048),
    # decode-sized batches
    (1, 2048, 8, 2, 8192), (32, 2048, 8, 2, 8192), (8, 2048, 64, 8, 1024), (64, 4096, 16, 2, 4096),
    (16, 7168, 256, 8, 2048), (128, 1024, 32, 1, 2048),
]
HELD_OUT_SHAPES = [
    (16384, 7168, 256, 8, 2048), (6144, 3072, 24, 3, 3072), (12288, 1536, 48, 6, 1536),
    (3072, 2048, 8, 2, 14336), (2048, 4096, 64, 4, 1024), (24576, 1024, 16, 2, 2048),
    (4, 2048, 8, 2, 8192), (24, 3072, 24, 3, 3072), (128, 2048, 64, 8, 1024), (8, 7168, 256, 8, 2048),
]


def main(argv=None):
    import argparse
    ap = argparse.ArgumentParser(description="Measure phase times on the GPU and fit the cost model.")
    ap.add_argument("--out", required=True, help="JSON file for the measured samples")
    ap.add_argument("--steps", type=int, default=10)
    args = ap.parse_args(argv)
    samples = []
    for shp in FIT_SHAPES + HELD_OUT_SHAPES:
        s = measure(*shp, steps=args.steps)
        print(f"{shp}: " + " ".join(f"{p}={s.phases_us[p]:.1f}" for p in PHASES), flush=True)
        samples.append(s)
    save_samples(samples, args.out)
    model = fit(samples[:len(FIT_SHAPES)])
    print("held-out MAPE %:", mape(model, samples[len(FIT_SHAPES):]), flush=True)


if __name__ == "__main__":
    main()
