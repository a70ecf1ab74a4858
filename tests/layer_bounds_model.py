"""A host model of the addresses k_moe_layer touches, for checking them
against their buffers on the CPU.

The model mirrors the kernel's index arithmetic function by function
(memory_bound_mxfp4_amd/csrc/layer.hip: launch_layer / launch_shape, the
workspace layout of api.hip's ws_layout, the unit loop of k_moe_layer, and
every unit body), thread by thread, for one call whose routing is given.
Every global access becomes (buffer, byte offset, bytes) and every LDS
access (region, byte offset, bytes); each is checked against the size of its
buffer or region.  Values that only decide arithmetic (weights, logits) are
not modelled; values that decide an address (the routing, the schedule the
device builds from it, the unit each workgroup takes) are.

It models the tiled layout at the shapes where FULL is false (H or I not a
multiple of 512: clamped and masked loads), which is where an index could
run past a buffer; the K3 shapes take the FULL branch of the same formulas.
When the kernel's indexing changes, this model has to follow it.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List

MAX_BATCH = 64
MAX_TOPK = 64
# kernel constants (layer.hip)
NT1, NTS1, NT2, NTS2, NTR2, CPL1, CPL2 = 16, 4, 256, 32, 128, 7, 6
MF_COLS, MF_NT1, MF_MT2 = 16, 64, 4
MF_NT2 = 128 * MF_MT2
MF_XS_FP4 = 512 * 2 + 16
MF_STAGE_BYTES = 2 * MF_COLS * MF_XS_FP4
CTRL_WORDS = 5 * 32  # five 128-byte lines: heads of the two work queues at lines 0 and 4
RT_F64_MIN_BATCH = 16


def align256(n):
    return (n + 255) & ~255


def topk_lds_words(tpl):
    return 4 * 64 * 2 + 4 * 64 * tpl * 2 + 4 + 2 * 64


def swz(g):
    return g ^ ((g >> 3) & 7)


def tile_off(g, s, C):
    return g * 16 * C * 17 + s * 16 * 272


def fc1_passes(S1, w):
    """layer.hip fc1_passes: batch-1 routed FC1 passes of wave w."""
    return (S1 - w + 3) // 4 if w < S1 else 0


def fc1_seg(w, p):
    """layer.hip Fc1Tile::seg: segment of wave w's pass p."""
    return w + 4 * p


def h_lo_offset(K):
    return ((K // 8 + 7) // 8) * 8


def scale_pos(SC, r, c):
    return r * 16 + (c & 3) * 4 + (c >> 2) if SC == 16 else r * SC + c


class OutOfBounds(AssertionError):
    pass


@dataclass
class Checker:
    sizes: Dict[str, int]
    count: int = 0
    where: str = ""

    def __call__(self, buf: str, off: int, nbytes: int):
        self.count += 1
        size = self.sizes[buf]
        if off < 0 or off + nbytes > size:
            raise OutOfBounds(f"{self.where}: {buf}[{off}:{off + nbytes}] outside [0, {size})")


@dataclass
class Shape:
    H: int
    I: int
    E: int
    k: int
    Is: int
    B: int


def blob_bytes(H, I):
    sz = [I * H // 2, I * H // 2, H * I // 2, I * H // 32, I * H // 32, H * I // 32]
    return sum(align256(s) for s in sz)


def ws_regions(sh: Shape):
    """api.hip ws_layout: region -> size in bytes (each 256-aligned)."""
    slots = sh.B * sh.k
    umax = min(slots, sh.E)
    n1 = max(sh.I, sh.Is)
    hflag_tiles = (n1 + 15) // 16
    return dict(ctrl=4 * CTRL_WORDS, logits_p=8 * sh.B * sh.E, idx_p=8 * slots, gate_p=8 * slots,
                active=4 * umax, row_off=4 * (umax + 1), rows=4 * slots, hs_p=8 * sh.B * max(sh.Is, 1),
                hr_p=8 * slots * sh.I, os_p=8 * sh.B * sh.H, or_p=8 * slots * sh.H, cg_off=4 * (umax + 1),
                hflag=8 * (umax + 1) * 4 * hflag_tiles), umax, hflag_tiles


def launch_shape(sh: Shape):
    """layer.hip launch_shape: (rg, full, xstride, hstride, lds, lds_h_off, lds_sched_off)."""
    H, I, E, k, Is, B = sh.H, sh.I, sh.E, sh.k, sh.Is, sh.B
    rg = 1 if B == 1 else 4
    full = (H % 512 == 0 and I % 512 == 0 and H % (32 * 8 * CPL1) == 0 and Is % (8 * 8 * CPL2) == 0
            and Is % NTS1 == 0 and H % NTR2 == 0 and H % NTS2 == 0)
    if B > 1:
        full = H % 512 == 0 and I % 512 == 0
    xstride = ((H // 8 + 7) // 8) * 8
    K2 = max(I, Is)
    hstride = ((K2 // 4 + 7) // 8) * 8
    if B == 1 and 2 * h_lo_offset(I) > hstride:
        hstride = 2 * h_lo_offset(I)
    x_bytes = 0 if B > 1 else rg * xstride * 16
    keys = topk_lds_words(4 if E <= 1024 else 16) * 4
    cnt = (3 * E + B * k) * 4
    xr = max(x_bytes, max(keys, cnt))
    if B > 1:
        xr = max(xr, MF_STAGE_BYTES)
    xr = align256(xr)
    hr = 0 if B > 1 else align256(2 * hstride * 16)  # batch 1: two h rows, alternating by unit
    slots = B * k
    umax = min(slots, E)
    lds = xr + hr + align256(4 * (3 * umax + 2 + slots))
    return dict(rg=rg, full=full, xstride=xstride, hstride=hstride, lds=lds, lds_h_off=xr, lds_sched_off=xr + hr)


@dataclass
class Params:
    sh: Shape
    ls: dict
    umax: int
    hflag_tiles: int
    n_rt_e: int = 0
    n_rb: int = 0
    n_rt: int = 0
    n_ro: int = 0
    n_sch: int = 0
    n_s1: int = 0
    T1: int = 0
    n_s2: int = 0
    n_r2: int = 0
    n_tile: int = 0
    mf_t1: int = 0
    mf_t1s: int = 0
    mf_t2: int = 0
    mf_t2s: int = 0
    mf_cgs: int = 0
    rt_f64: bool = False


def params(sh: Shape) -> Params:
    """layer.hip launch_layer: the unit counts of the queue."""
    _, umax, tiles = ws_regions(sh)
    p = Params(sh, launch_shape(sh), umax, tiles)
    H, I, E, k, Is, B = sh.H, sh.I, sh.E, sh.k, sh.Is, sh.B
    p.rt_f64 = B > RT_F64_MIN_BATCH
    p.n_rt_e = (E + 15) // 16 if p.rt_f64 else (E + 3) // 4
    p.n_rb = (B + 15) // 16 if p.rt_f64 else ((B + 7) // 8 if B > 1 else 1)
    p.n_rt = p.n_rt_e * p.n_rb
    p.n_ro = B
    p.n_sch = 1 if B > 1 else 0
    p.n_s1 = (Is + NTS1 - 1) // NTS1 if Is > 0 else 0
    p.T1 = (I + NT1 - 1) // NT1
    p.n_s2 = (H + NTS2 - 1) // NTS2 if Is > 0 else 0
    p.n_r2 = (H + NTR2 - 1) // NTR2
    p.n_tile = (H + NT2 - 1) // NT2
    p.mf_t1 = (I + MF_NT1 - 1) // MF_NT1
    p.mf_t1s = (Is + 15) // 16
    p.mf_t2 = (H + MF_NT2 - 1) // MF_NT2
    p.mf_t2s = (H + 127) // 128
    p.mf_cgs = (B + MF_COLS - 1) // MF_COLS
    if B > 1:
        p.n_s1 = p.mf_cgs * p.mf_t1s if Is > 0 else 0
        p.n_s2 = p.mf_cgs * p.mf_t2s if Is > 0 else 0
    return p


@dataclass
class Schedule:
    """The expert-gathered schedule build_schedule publishes (or, at batch 1,
    the one cache_schedule makes from the slots)."""
    U: int
    active: List[int]
    row_off: List[int]
    rows: List[int]
    cg_off: List[int]


def build_schedule(sh: Shape, idx: List[List[int]]) -> Schedule:
    E, k, B = sh.E, sh.k, sh.B
    ids = [min(max(int(idx[s // k][s % k]), 0), E - 1) for s in range(B * k)]
    if B == 1:
        return Schedule(k, ids, list(range(k + 1)), list(range(k)), [])
    cnt = [0] * E
    for e in ids:
        cnt[e] += 1
    active, row_off, cg_off, start = [], [], [], [0] * E
    pr = pc = 0
    for e in range(E):
        start[e] = pr
        if cnt[e]:
            active.append(e)
            row_off.append(pr)
            cg_off.append(pc)
        pr += cnt[e]
        pc += (cnt[e] + 15) >> 4
    row_off.append(pr)
    cg_off.append(pc)
    rows = [0] * (B * k)
    for s in range(B * k):  # any order within an expert: every order is covered by the bounds
        rows[start[ids[s]]] = s
        start[ids[s]] += 1
    return Schedule(len(active), active, row_off, rows, cg_off)


def _lanes():
    for t in range(256):
        yield t, t >> 6, t & 63


def check_call(sh: Shape, idx: List[List[int]], bias: bool = False) -> int:
    """Walk every unit of one call with routing `idx` ([B][k]); raise
    OutOfBounds at the first access outside its buffer.  Returns the number of
    accesses checked."""
    p = params(sh)
    H, I, E, k, Is, B = sh.H, sh.I, sh.E, sh.k, sh.Is, sh.B
    regions, umax, tiles = ws_regions(sh)
    ls = p.ls
    nb = blob_bytes(H, I)
    sizes = dict(regions)
    sizes.update(x=2 * B * H, wr=2 * E * H, bias=4 * E if bias else 0, sg=2 * Is * H, su=2 * Is * H,
                 sd=2 * H * Is, experts=E * nb, residual=4 * B * H, idx=4 * B * k, gate=4 * B * k,
                 lds=ls["lds"], lds_slot=4 * MAX_BATCH, lds_gates=4 * MAX_TOPK, lds_red=4 * 4 * 4 * 16 * 2)
    chk = Checker(sizes)
    sched = build_schedule(sh, idx)
    xs = 0
    hs = ls["lds_h_off"]
    sc = ls["lds_sched_off"]
    # the LDS copy of the schedule (cache_schedule): a | ro | rw | cgo
    a_off, ro_off = sc, sc + 4 * umax
    rw_off = ro_off + 4 * (umax + 1)
    cgo_off = rw_off + 4 * B * k
    MF = B > 1
    U = sched.U
    for i in range(U):
        chk.where = "cache_schedule"
        chk("lds", a_off + 4 * i, 4)
        chk("lds", ro_off + 4 * i, 4)
        if MF:
            chk("lds", cgo_off + 4 * i, 4)
            chk("active", 4 * i, 4)
            chk("row_off", 4 * i, 4)
            chk("cg_off", 4 * i, 4)
    chk("lds", ro_off + 4 * U, 4)
    for s in range(B * k):
        chk("lds", rw_off + 4 * s, 4)
        if not MF:
            chk("idx_p", 8 * s, 8)
    if MF:
        chk("lds", cgo_off + 4 * U, 4)
        chk("row_off", 4 * U, 4)
        chk("cg_off", 4 * U, 4)
        for s in range(B * k):
            chk("rows", 4 * s, 4)

    # ---- front units ----
    for u in range(p.n_rt):
        chk.where = f"router unit {u}"
        if not MF:
            C = H // 8
            for t, w, lane in _lanes():
                e = 4 * u + w
                for c0 in range(lane, C, 64 * 14):
                    for i in range(14):
                        c = min(c0 + 64 * i, C - 1)
                        chk("wr", 2 * (min(e, E - 1) * H + 8 * c), 16)
                        chk("x", 2 * 8 * c, 16)
                if e < E and lane == 0:
                    if bias:
                        chk("bias", 4 * e, 4)
                    chk("logits_p", 8 * e, 8)
        elif p.rt_f64:  # router_f64_unit
            et, rt = u % p.n_rt_e, u // p.n_rt_e
            e0, b0 = 16 * et, 16 * rt
            C = H // 8
            NCH = (C + 3) // 4
            per = (NCH + 3) // 4
            for t, w, lane in _lanes():
                r, q = lane & 15, lane >> 4
                ch0, ch1 = w * per, min(NCH, w * per + per)
                gran = lambda ch: min(4 * min(ch, NCH - 1) + q, C - 1)
                chunks = list(range(ch0, ch0 + 8)) + list(range(ch0 + 8, ch1))
                for ch in chunks:
                    g = gran(ch)
                    chk("wr", 2 * (min(e0 + r, E - 1) * H + 8 * g), 16)
                    chk("x", 2 * (min(b0 + r, B - 1) * H + 8 * g), 16)
                for i in range(4):
                    chk("lds", 8 * ((w * 16 + 4 * i + q) * 16 + r), 8)
                row, col = t >> 4, t & 15
                for ww in range(4):
                    chk("lds", 8 * (256 * ww + t), 8)
                if e0 + row < E and b0 + col < B:
                    if bias:
                        chk("bias", 4 * (e0 + row), 4)
                    chk("logits_p", 8 * ((b0 + col) * E + e0 + row), 8)
        else:
            eg, rb = u % p.n_rt_e, u // p.n_rt_e
            e0, b0 = 4 * eg, 8 * rb
            nr = min(8, B - b0)
            C = H // 8
            Q = (C + 3) // 4
            J = (Q + 63) // 64
            for t, w, lane in _lanes():
                c_lo = w * Q
                for j in range(J):
                    c = min(c_lo + lane + 64 * j, C - 1)
                    for e in range(4):
                        chk("wr", 2 * (min(e0 + e, E - 1) * H + 8 * c), 16)
                    for r in range(8):
                        chk("x", 2 * ((b0 + min(r, nr - 1)) * H + 8 * c), 16)
                if (lane & 1) == 0:
                    chk("lds_red", 8 * (w * 32 + (lane >> 1)), 8)
                if t < 32:
                    e, r = e0 + t // 8, t % 8
                    for ww in range(4):
                        chk("lds_red", 8 * (ww * 32 + t), 8)
                    if e < E and r < nr:
                        chk("logits_p", 8 * ((b0 + r) * E + e), 8)
    for b in range(p.n_ro):
        chk.where = f"routing unit {b}"
        _topk(chk, sh, b, xs)
    if MF:
        chk.where = "schedule unit"
        for s in range(B * k):
            chk("idx_p", 8 * s, 8)
        for e in range(E):
            chk("lds", xs + 8 * e, 8)  # row set (8 bytes an expert)
            chk("lds", xs + 4 * (2 * E + e), 4)  # start
        for s in range(B * k):
            chk("lds", xs + 4 * (3 * E + s), 4)  # slot ids
        chk("ctrl", 4 * 96, 8)
    for u in range(p.n_s1):
        chk.where = f"shared FC1 unit {u}"
        if MF:
            _mf_sh1(chk, p, u // p.mf_t1s, u % p.mf_t1s)
        else:
            _shared_fc1_b1(chk, p, u, xs)

    # ---- routed and tail units ----
    if MF:
        NCG = sched.cg_off[U]
        for rel in range(NCG * p.mf_t1):
            gc = rel // p.mf_t1
            ae = _find_expert(sched, gc)
            chk.where = f"routed FC1 unit {rel} (expert {sched.active[ae]}, column group {gc - sched.cg_off[ae]})"
            _mf_fc1(chk, p, sched, ae, min(gc - sched.cg_off[ae], 3), rel % p.mf_t1, nb)
        for rel in range(p.n_s2):
            chk.where = f"shared FC2 unit {rel}"
            _mf_fc2(chk, p, sched, -1, rel // p.mf_t2s, rel % p.mf_t2s, nb)
        for rel in range(NCG * p.mf_t2):
            gc = rel // p.mf_t2
            ae = _find_expert(sched, gc)
            chk.where = f"routed FC2 unit {rel} (expert {sched.active[ae]}, column group {gc - sched.cg_off[ae]})"
            _mf_fc2(chk, p, sched, ae, min(gc - sched.cg_off[ae], 3), rel % p.mf_t2, nb)
    else:
        for rel in range(U * p.T1):
            chk.where = f"routed FC1 unit {rel}"
            _routed_fc1_b1(chk, p, sched, rel // p.T1, rel % p.T1, nb, xs)
        for rel in range(p.n_s2):
            chk.where = f"shared FC2 unit {rel}"
            _shared_fc2_b1(chk, p, rel, hs)
        for rel in range(U * p.n_r2):
            chk.where = f"routed FC2 unit {rel}"
            _routed_fc2_b1(chk, p, sched, rel // p.n_r2, rel % p.n_r2, nb, hs)
    for rel in range(B * p.n_tile):
        chk.where = f"combine unit {rel}"
        _combine(chk, p, rel // p.n_tile, rel % p.n_tile)
    chk.where = "exit"
    chk("ctrl", 0, 4)
    chk("ctrl", 4 * 32, 4)
    chk("ctrl", 4 * 64, 4)
    chk("ctrl", 4 * 128, 4)
    return chk.count


def _find_expert(sched: Schedule, gc: int) -> int:
    lo, hi = 0, sched.U - 1
    while lo < hi:
        mid = (lo + hi + 1) >> 1
        if sched.cg_off[mid] <= gc:
            lo = mid
        else:
            hi = mid - 1
    return lo


def _topk(chk, sh: Shape, b: int, cand: int):
    """moe_device.h topk_row_wg (TPL 4 for E <= 1024): the logits polls and
    every LDS word of `cand`.  Survivor counts up to every entry of the row
    are covered (the bound for all-equal keys is n = G)."""
    E, k = sh.E, sh.k
    TPL = 4 if E <= 1024 else 16
    Q = (E + 3) // 4
    G = 1
    while G < k:
        G <<= 1
    bs = 64 // G
    gbest, surv = cand, cand + 4 * (4 * 64 * 2)
    nsurv = surv + 4 * (4 * 64 * TPL * 2)
    out = nsurv + 4 * 4
    chk("lds", nsurv, 4)
    for t, w, lane in _lanes():
        e0, e1 = w * Q, min(E, w * Q + Q)
        mine = max(0, min(TPL, (e1 - e0 - lane + 63) // 64))
        for i in range(max(mine, 1)):
            chk("logits_p", 8 * (b * E + min(e0 + lane + 64 * i, E - 1)), 8)
        if (lane & (bs - 1)) == 0:
            chk("lds", gbest + 8 * (w * 64 + lane // bs), 8)
        if lane < G:
            for ww in range(4):
                chk("lds", gbest + 8 * (64 * ww + lane), 8)
    for n in (1, k, min(E, 64), min(E, 4 * 64 * TPL)):  # survivor counts, up to all entries
        for pos in range(n):
            chk("lds", surv + 4 * (2 * pos), 8)
        lp = 2 if n <= 64 else (1 if n <= 128 else 0)
        span = (((n + (1 << lp) - 1) >> lp) + 1) & ~1
        for base in range(0, n << lp, 256):
            for t in range(256):
                tt = base + t
                sidx, part = tt >> lp, tt & ((1 << lp) - 1)
                if sidx >= n:
                    continue
                j0 = min(n, part * span)
                j1 = min(n, j0 + span)
                j = j0
                while j + 4 <= j1:
                    chk("lds", surv + 4 * (2 * j), 16)
                    chk("lds", surv + 4 * (2 * j + 4), 16)
                    j += 4
                while j < j1:
                    chk("lds", surv + 4 * (2 * j), 8)
                    j += 1
        for r in range(min(n, k)):
            chk("lds", out + 4 * (2 * r), 8)
    for lane in range(k):
        chk("lds", out + 4 * (2 * lane), 8)
        chk("idx", 4 * (b * k + lane), 4)
        chk("gate", 4 * (b * k + lane), 4)
        chk("idx_p", 8 * (b * k + lane), 8)
        chk("gate_p", 8 * (b * k + lane), 8)


def _shared_fc1_b1(chk, p: Params, t: int, xs: int):
    sh = p.sh
    H, Is = sh.H, sh.Is
    n_begin, n_end = t * NTS1, min(Is, t * NTS1 + NTS1)
    C8 = H // 8
    nseg = (C8 + 32 * CPL1 - 1) // (32 * CPL1)
    chk("lds_slot", 0, 4)
    for c in range(H // 8):  # stage_x (one row)
        chk("lds", xs + 16 * (swz(c)), 16)
        chk("x", 16 * c, 16)
    for tt, w, lane in _lanes():
        half = lane >> 5
        n0 = n_begin + w
        nrows = (n_end - n0 + 3) // 4 if n0 < n_end else 0
        for pp in range(nrows * nseg):
            i, s = pp // nseg, pp % nseg
            n = n0 + 4 * i
            l = lane & 31
            c0 = s * 32 * CPL1 + l
            for ci in range(CPL1):
                c = min(c0 + 32 * ci, C8 - 1)
                chk("su" if half else "sg", 2 * (n * H + 8 * c), 16)
                chk("lds", xs + 16 * swz(c), 16)
            if s == nseg - 1 and lane == 0:
                chk("hs_p", 8 * (0 * Is + n), 8)


def _load_tile(chk, buf, t, SC, lane):
    r, q = lane & 15, lane >> 4
    for kb in range(4):
        c = min(4 * kb + q, SC - 1)
        chk(buf, t + c * 256 + r * 16, 16)
        chk(buf, t + SC * 256 + scale_pos(SC, r, c), 1)


def _routed_fc1_b1(chk, p: Params, sched: Schedule, a: int, g: int, nb: int, xs: int):
    sh = p.sh
    H, I = sh.H, sh.I
    slot = sched.rows[sched.row_off[a]]
    blob = sched.active[a] * nb
    C1 = H // 32
    S1 = (C1 + 15) // 16
    for c in range(H // 8):
        chk("lds", xs + 16 * swz(c), 16)
        chk("x", 16 * c, 16)
    # Passes 0 and 1 of a wave with an even pass count may be issued by the
    # unit before (the hand-on of fc1_unit_b1) when that was a routed FC1 unit
    # too: the same addresses, computed from the same schedule entry.
    for t, w, lane in _lanes():
        P = fc1_passes(S1, w)
        q = lane >> 4
        for pp in range(P):
            s = fc1_seg(w, pp)
            SC = min(16, C1 - 16 * s)
            gt = blob + 2 * tile_off(g, s, C1)
            _load_tile(chk, "experts", gt, SC, lane)
            _load_tile(chk, "experts", gt + SC * 272, SC, lane)
            for i in range(16):
                c = 4 * (i >> 2) + q
                chk("lds", xs + 16 * swz((16 * s + min(c, SC - 1)) * 4 + (i & 3)), 16)
        if (lane & 15) == 0:
            for i in range(4):
                chk("lds_red", 4 * (((w * 4 + 0) * 16 + 4 * (lane >> 4) + i) * 2), 8)
        if t < 16:
            chk("hr_p", 8 * (slot * I + 16 * g + t), 8)


def _shared_fc2_b1(chk, p: Params, v: int, hs: int):
    sh = p.sh
    H, Is = sh.H, sh.Is
    hstride = p.ls["hstride"]
    m_begin, m_end = v * NTS2, min(H, v * NTS2 + NTS2)
    C8 = Is // 8
    nseg = (C8 + 8 * CPL2 - 1) // (8 * CPL2)
    groups = (m_end - m_begin + 31) // 32
    for e in range(Is):  # stage_h
        chk("hs_p", 8 * e, 8)
        chk("lds", hs + 4 * ((0 * hstride + swz(e >> 2)) * 4 + (e & 3)), 4)
    for t, w, lane in _lanes():
        for pp in range(groups * nseg if m_begin < m_end else 0):
            grp, s = pp // nseg, pp % nseg
            m_raw = m_begin + (w + 4 * grp) * 8 + (lane >> 3)
            m = min(m_raw, m_end - 1)
            l = lane & 7
            c0 = s * 8 * CPL2 + l
            for ci in range(CPL2):
                c = min(c0 + 8 * ci, C8 - 1)
                chk("sd", 2 * (m * Is + 8 * c), 16)
                chk("lds", hs + 16 * swz(2 * c), 16)
                chk("lds", hs + 16 * swz(2 * c + 1), 16)
            if s == nseg - 1 and l == 0 and m_raw < m_end:
                chk("os_p", 8 * m_raw, 8)


def _routed_fc2_b1(chk, p: Params, sched: Schedule, a: int, v: int, nb: int, hs: int):
    sh = p.sh
    H, I = sh.H, sh.I
    slot = sched.rows[sched.row_off[a]]
    C1, C2 = H // 32, I // 32
    S2 = (C2 + 15) // 16
    down = sched.active[a] * nb + 2 * I * C1 * 17
    G = H // 16
    hlo = h_lo_offset(I)
    for hb in (hs, hs + 16 * p.ls["hstride"]):  # either of the two h rows (by unit-loop iteration)
        _routed_fc2_b1_h(chk, p, sched, a, v, nb, hb, slot, down, hlo)


def _routed_fc2_b1_h(chk, p: Params, sched: Schedule, a: int, v: int, nb: int, hs: int, slot: int, down: int,
                     hlo: int):
    sh = p.sh
    H, I = sh.H, sh.I
    C2 = I // 32
    S2 = (C2 + 15) // 16
    G = H // 16
    # the staged row (hi granules, then lo at hlo) stays inside the h region, clear of the schedule
    assert p.ls["lds_h_off"] <= hs and hs + 16 * 2 * hlo <= p.ls["lds_sched_off"]
    for e in range(I):  # stage_h_split (at the unit's start, or at the end of the unit before)
        chk("hr_p", 8 * (slot * I + e), 8)
        chk("lds", hs + 2 * (swz(e >> 3) * 8 + (e & 7)), 2)
        chk("lds", hs + 2 * ((hlo + swz(e >> 3)) * 8 + (e & 7)), 2)
    for t, w, lane in _lanes():
        g0 = 8 * v + w
        ng = (2 if g0 + 4 < G else 1) if g0 < G else 0
        g0c = min(g0, G - 1)
        q = lane >> 4
        for s in range(S2 if ng > 0 else 0):
            SC = min(16, C2 - 16 * s)
            for tt in range(2):
                _load_tile(chk, "experts", down + tile_off(g0c + 4 * (tt if tt < ng else 0), s, C2), SC, lane)
            for i in range(16):
                c = 4 * (i >> 2) + q
                chk("lds", hs + 16 * ((lane & 1) * hlo + swz((16 * s + min(c, SC - 1)) * 4 + (i & 3))), 16)
        if (lane & 15) == 0:  # regroup_rows + st_pair2_f32: rows 8 h + 2 q, + 1 of the tile
            for tt in range(ng):
                for h in range(2):
                    chk("or_p", 8 * (slot * H + 16 * (g0 + 4 * tt) + 8 * h + 2 * (lane >> 4)), 16)


def _combine(chk, p: Params, b: int, t: int):
    sh = p.sh
    H, k = sh.H, sh.k
    for tid in range(k):
        chk("gate_p", 8 * (b * k + tid), 8)
        chk("lds_gates", 4 * tid, 4)
    for tid in range(256):
        m = t * NT2 + tid
        if m >= H:
            continue
        chk("residual", 4 * (b * H + m), 4)
        if sh.Is > 0:
            chk("os_p", 8 * (b * H + m), 8)
        for j in range(k):
            chk("or_p", 8 * ((b * k + j) * H + m), 8)


def _load_cols(chk, p: Params, sched: Schedule, a: int, cg: int):
    B = p.sh.B
    if a < 0:
        n = min(MF_COLS, B - MF_COLS * cg)
        slots = [MF_COLS * cg + i for i in range(n)]
    else:
        n = min(MF_COLS, sched.row_off[a + 1] - (sched.row_off[a] + MF_COLS * cg))
        slots = [sched.rows[sched.row_off[a] + MF_COLS * cg + i] for i in range(n)]
    for i in range(n):
        chk("lds_slot", 4 * i, 4)
    return slots


def _hflag(chk, p: Params, ex: int, cg: int, t: int):
    chk("hflag", 8 * ((ex * 4 + cg) * p.hflag_tiles + t), 8)


def _mf_sh1(chk, p: Params, cg: int, g: int):
    sh = p.sh
    H, Is, B = sh.H, sh.Is, sh.B
    slots = _load_cols(chk, p, None, -1, cg)
    nc = len(slots)
    S = (H + 127) // 128
    for t, w, lane in _lanes():
        r, q = lane & 15, lane >> 4
        P = (S - w + 3) // 4 if w < S else 0
        xrow = slots[r if r < nc else 0]
        for pp in range(P):
            s = w + 4 * pp
            n = min(16 * g + r, Is - 1)
            for j in range(4):
                k0 = min(s * 128 + 32 * j + 8 * q, H - 8)
                chk("sg", 2 * (n * H + k0), 16)
                chk("su", 2 * (n * H + k0), 16)
                chk("x", 2 * (xrow * H + k0), 16)
        for i in range(4):
            for m in range(2):
                chk("lds", 4 * (((w * 2 + m) * 16 + 4 * q + i) * 16 + r), 4)
        row, col = t >> 4, t & 15
        for ww in range(4):
            for m in range(2):
                chk("lds", 4 * (((ww * 2 + m) * 16 + row) * 16 + col), 4)
        n = 16 * g + row
        if col < nc and n < Is:
            chk("hs_p", 4 * (slots[col] * Is + n), 4)
    _hflag(chk, p, p.umax, cg, g)


def _mf1_load_fp4(chk, p, blob, g, s, lane):
    C1 = p.sh.H // 32
    SC = min(16, C1 - 16 * s)
    gt = blob + 2 * tile_off(g, s, C1)
    _load_tile(chk, "experts", gt, SC, lane)
    _load_tile(chk, "experts", gt + SC * 272, SC, lane)


def _mf_fc1(chk, p: Params, sched: Schedule, a: int, cg: int, t: int, nb: int):
    sh = p.sh
    H, I, k = sh.H, sh.I, sh.k
    N = I
    blob = sched.active[a] * nb
    S = (H // 32 + 15) // 16
    slots = _load_cols(chk, p, sched, a, cg)
    nc = len(slots)
    XF = H * 2 + 16
    KS, XS = 512, 512 * 2 + 16
    C1 = H // 32
    narrow = nc * XF <= MF_STAGE_BYTES
    if narrow:
        CPC = H // 8
        total = nc * CPC
        for ch in range(total):
            c, j = ch // CPC, ch % CPC
            chk("x", 2 * ((slots[c] // k) * H + 8 * j), 16)
            chk("lds", c * XF + 16 * j, 16)
    else:
        CPC = KS * 2 // 16
        for s in range(S):
            for ch in range(MF_COLS * CPC):
                c, j = ch // CPC, ch % CPC
                k0 = s * KS + 8 * j
                if c < nc and k0 < H:
                    chk("x", 2 * ((slots[c] // k) * H + k0), 16)
                chk("lds", (s & 1) * MF_COLS * XS + c * XS + 16 * j, 16)
    for tt, w, lane in _lanes():
        r, q = lane & 15, lane >> 4
        g = 4 * t + w
        gl = min(g, (N + 15) // 16 - 1)
        for s in range(S):
            _mf1_load_fp4(chk, p, blob, gl, s, lane)
            SC = min(16, C1 - 16 * s)
            for i in range(16):
                kb, d = i >> 2, i & 3
                c = 4 * kb + q
                dd = d if c < SC else 0
                if narrow:
                    col = r if r < nc else 0
                    chk("lds", col * XF + s * KS * 2 + (128 * kb + 32 * q + 8 * dd) * 2, 16)
                else:
                    chk("lds", (s & 1) * MF_COLS * XS + r * XS + (128 * kb + 32 * q + 8 * dd) * 2, 16)
        n0 = 16 * g + 4 * q
        if n0 < N and r < nc:
            chk("hr_p", 4 * (slots[r] * N + n0), 16)
    _hflag(chk, p, a, cg, t)


def _mf_fc2(chk, p: Params, sched: Schedule, a: int, cg: int, t: int, nb: int):
    sh = p.sh
    H, I, Is = sh.H, sh.I, sh.Is
    FP4 = a >= 0
    K = I if FP4 else Is
    G = H // 16
    down = sched.active[a] * nb + 2 * I * (H // 32) * 17 if FP4 else 0
    S = (K // 32 + 15) // 16 if FP4 else (K + 127) // 128
    MT2 = MF_MT2 if FP4 else 1
    MT = min(MT2, (G - 8 * MT2 * t + 7) // 8)
    slots = _load_cols(chk, p, sched, a, cg)
    nc = len(slots)
    XF = K * 2 + 16
    narrow = 2 * (nc if nc <= 8 else 1024) * XF <= MF_STAGE_BYTES
    ntile = (K + MF_NT1 - 1) // MF_NT1 if FP4 else (K + 15) // 16
    for ti in range(ntile):
        _hflag(chk, p, a if FP4 else p.umax, cg, ti)
    hsrc = "hr_p" if FP4 else "hs_p"
    hsrc_elem = 4  # fp32 view of the pair arrays

    def stage(k0, KE, ncols, XS, lo_off):
        HP = KE // 2
        for e in range(ncols * HP):
            c, j = e // HP, e % HP
            kk = k0 + 2 * j
            if c < nc and kk < K:
                chk(hsrc, hsrc_elem * (slots[c] * K + kk), 8)
            chk("lds", c * XS + 4 * j, 4)
            chk("lds", lo_off + c * XS + 4 * j, 4)

    def load(gt, s, lane):
        r, q = lane & 15, lane >> 4
        if FP4:
            C2 = I // 32
            SC = min(16, C2 - 16 * s)
            for tt in range(2):
                _load_tile(chk, "experts", down + tile_off(gt[tt], s, C2), SC, lane)
        else:
            for tt in range(2):
                m = min(16 * gt[tt] + r, H - 1)
                for j in range(4):
                    k0 = min(s * 128 + 32 * j + 8 * q, Is - 8)
                    chk("sd", 2 * (m * Is + k0), 16)

    def groups(mt, w):
        return (min(8 * (MT2 * t + mt) + w, G - 1), min(8 * (MT2 * t + mt) + w + 4, G - 1))

    def math_reads(s, hb, lo, hoff, lane, live):
        q = lane >> 4
        if FP4:
            C2 = I // 32
            SC = min(16, C2 - 16 * s)
            for i in range(16):
                kb, d = i >> 2, i & 3
                c = 4 * kb + q
                bv = live and c < SC
                off = hoff + ((128 * kb + 32 * q + 8 * d) * 2 if bv else 0)
                chk("lds", hb + off, 16)
                chk("lds", lo + off, 16)
        else:
            for j in range(4):
                ok = s * 128 + 32 * j + 8 * q < Is
                off = hoff + ((32 * j + 8 * q) * 2 if ok else 0)
                chk("lds", hb + off, 16)
                chk("lds", lo + off, 16)

    def emit(mt, w, lane):
        r, q = lane & 15, lane >> 4
        if r < nc:
            for tt in range(2):
                g = 8 * (MT2 * t + mt) + w + 4 * tt
                if g < G:
                    for h in range(2):  # regroup_rows + st_pair2_f32
                        chk("or_p" if FP4 else "os_p", 8 * (slots[r] * H + 16 * g + 8 * h + 2 * q), 16)

    if narrow:
        KS = 512 if FP4 else 128
        stage(0, K, nc, XF, nc * XF)
        for tt, w, lane in _lanes():
            r = lane & 15
            cc = r & 7  # packed hi + lo: lanes r < 8 read the hi half of column r, r >= 8 the lo half of r - 8
            live = cc < nc
            hcol = (cc if live else 0) * XF + (nc * XF if r >= 8 else 0)
            for ps in range(MT * S):
                mt, sg = ps // S, ps % S
                load(groups(mt, w), sg, lane)
                math_reads(sg, hcol, hcol, sg * KS * 2, lane, live)
                if sg == S - 1:
                    emit(mt, w, lane)
    else:
        XS = 512 * 2 + 16
        NCH = (K + 511) // 512
        for c in range(NCH):
            stage(c * 512, 512, MF_COLS, XS, MF_COLS * XS)
            for tt, w, lane in _lanes():
                r = lane & 15
                for j in range(4):
                    seg = c if FP4 else 4 * c + j
                    if seg < S and (j < MT if FP4 else True):
                        load(groups(j if FP4 else 0, w), seg, lane)
                        math_reads(seg, r * XS, MF_COLS * XS + r * XS, 0 if FP4 else j * 256, lane, True)
        for tt, w, lane in _lanes():
            for i in range(MT):
                emit(i, w, lane)
