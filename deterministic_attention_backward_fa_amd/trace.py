"""Per-tile phase timeline of the main kernel (the optional device trace).

`collect` runs one attn_bwd_deterministic call with a trace buffer; every
workgroup's wave 0 records (s_memtime, phase | tile << 8 | item << 32) at the
phase boundaries listed in detattn_trace_phase_t. `summarize` turns the
records into the mean share of each phase per tile, which shows where a
schedule's time goes on the hardware (compute, waiting for the dQ tile's turn,
accumulator adds, barriers).
"""
import numpy as np
import torch

PHASES = {0: "tile_top", 1: "ds_ready", 2: "dq_done", 3: "turn", 4: "adds_issued", 5: "tile_end", 6: "seg_begin",
          7: "seg_end", 8: "wg_start", 9: "registered"}
# consecutive phase pairs inside one tile, and the name of the interval. A
# tile whose turn had already come at its top reads the accumulator right
# after the dS^T barrier (phase 3 before phase 2); the others wait after the
# dQ MFMAs.
INTERVALS = [
    (0, 1, "S,dP MFMA + P,dS VALU + dS^T store"),
    (1, 2, "barrier + dQ MFMA issue"),
    (2, 3, "wait for the dQ tile's turn"),
    (3, 4, "accumulator adds issued"),
    (1, 3, "barrier (turn already come)"),
    (3, 2, "accumulator reads + dQ MFMA issue"),
    (2, 4, "dV,dK MFMA issue up to the adds"),
    (4, 5, "dV,dK MFMA issue"),
    (5, 0, "drain + barrier + publish (to next tile)"),
]


def collect(da, tensors, causal, schedule, records=4096, **opts):
    q, k, v, o, do, lse = tensors
    B, H, S, D = q.shape
    plan = da.detattn_bwd_plan(B, H, S, D, causal, schedule, **opts)
    buf = torch.zeros(plan["grid"] * records * 2, dtype=torch.int64, device=q.device)
    ws = da.alloc_workspace(B, H, S, D)
    da.attn_bwd_deterministic(q, k, v, o, do, lse, causal=causal, schedule=schedule, workspace=ws, trace=buf,
                              trace_records=records, **opts)
    torch.cuda.synchronize()
    return buf.view(plan["grid"], records, 2).cpu().numpy(), plan


# Gantt symbols per interval (phase a -> phase b); the rest is compute ('#')
_GANTT = {(2, 3): "w", (5, 7): "e", (7, 6): "e", (6, 0): "e", (8, 9): "s", (9, 6): "s", (8, 6): "s"}
_PRIORITY = {" ": 0, "#": 1, "e": 2, "s": 2, "w": 3}


def summarize(recs):
    """Mean ticks per tile of each interval, over every workgroup's complete tiles."""
    sums = {name: [] for _, _, name in INTERVALS}
    spans = []
    for wg in range(recs.shape[0]):
        r = recs[wg]
        r = r[r[:, 0] != 0]
        if len(r) < 2:
            continue
        t = r[:, 0].astype(np.int64)
        ph = (r[:, 1] & 0xFF).astype(np.int64)
        spans.append(t[-1] - t[0])
        for x in range(len(r) - 1):
            for a, b, name in INTERVALS:
                if ph[x] == a and ph[x + 1] == b:
                    sums[name].append(t[x + 1] - t[x])
    # mean ticks per tile: each interval's total over all tiles (intervals of
    # only one of the two turn paths are weighted by how often that path runs)
    n_tiles = max(1, sum(len(v) for a, b, v in ((a, b, sums[n]) for a, b, n in INTERVALS) if (a, b) == (0, 1)))
    out = {name: (float(np.sum(v)) / n_tiles if v else 0.0) for name, v in sums.items()}
    total = sum(out.values())
    # tile period (top to top) and how many tiles found their turn already come
    # at the dS^T barrier (turn recorded before the dQ MFMAs)
    periods, early, late = [], 0, 0
    for wg in range(recs.shape[0]):
        r = recs[wg]
        r = r[r[:, 0] != 0]
        t = r[:, 0].astype(np.int64)
        ph = (r[:, 1] & 0xFF).astype(np.int64)
        tops = t[ph == 0]
        if len(tops) > 1:
            periods.extend(np.diff(tops).tolist())
        for x in range(len(r) - 1):
            if ph[x] == 1:
                early += int(ph[x + 1] == 3)
                late += int(ph[x + 1] == 2)
    # each workgroup's traced span split into tile work, column switches
    # (dK/dV stores, the next K/V) and start-up (registration, first K/V)
    split = {"tiles": 0, "column switch": 0, "start-up": 0}
    for wg in range(recs.shape[0]):
        r = recs[wg]
        r = r[r[:, 0] != 0]
        t = r[:, 0].astype(np.int64)
        ph = (r[:, 1] & 0xFF).astype(np.int64)
        if not np.any(ph == 0):
            continue  # no ring: the workgroup only registered
        for x in range(len(r) - 1):
            kind = _GANTT.get((int(ph[x]), int(ph[x + 1])), "#")
            key = "column switch" if kind == "e" else "start-up" if kind == "s" else "tiles"
            split[key] += int(t[x + 1] - t[x])
    span_total = sum(split.values())
    return {"mean_ticks_per_tile": total, "share": {k: (v / total if total else 0.0) for k, v in out.items()},
            "span_share": {k: (v / span_total if span_total else 0.0) for k, v in split.items()},
            "ticks": out, "workgroups": len(spans),
            "tile_period_median": float(np.median(periods)) if periods else 0.0,
            "early_turn_fraction": early / (early + late) if early + late else 0.0}


def gantt(recs, width=100, max_rows=64):
    """Text timeline of the traced workgroups: one row per workgroup, one column
    per 1/width of the traced span. '#' computing a tile, 'w' waiting for a dQ
    tile's turn, 'e' switching columns (dK/dV stores, the next K/V), ' ' idle.
    A column shows the most telling state that falls into it (w > e > #).
    The cycle counters of different compute units are not synchronized, so
    every row starts at its workgroup's first record: the workgroups of the
    persistent grid all start at launch, up to the launch skew."""
    # workgroups that ran at least one tile (those without a ring only register)
    rows = [wg for wg in range(recs.shape[0])
            if np.any((recs[wg][:, 0] != 0) & ((recs[wg][:, 1] & 0xFF) == 0))][:max_rows]
    if not rows:
        return ""
    spans = []
    for wg in rows:
        r = recs[wg]
        r = r[r[:, 0] != 0]
        spans.append(int(r[-1, 0]) - int(r[0, 0]))
    scale = width / max(1, max(spans))
    lines = []
    for wg in rows:
        r = recs[wg]
        r = r[r[:, 0] != 0]
        t0 = int(r[0, 0])
        t = r[:, 0].astype(np.int64)
        ph = (r[:, 1] & 0xFF).astype(np.int64)
        cells = [" "] * width
        for x in range(len(r) - 1):
            sym = _GANTT.get((int(ph[x]), int(ph[x + 1])), "#")
            a = min(width - 1, int((t[x] - t0) * scale))
            b = min(width - 1, int((t[x + 1] - t0) * scale))
            for c in range(a, b + 1):
                if _PRIORITY[sym] > _PRIORITY[cells[c]]:
                    cells[c] = sym
        lines.append(f"{wg:4d} |{''.join(cells)}|")
    return "\n".join(lines)
