"""The chunked-prefill kernel's LDS-stage protocol, checked on the host.

The kernel stages K and V tiles in a ring of LDS stages filled by DMAs that
the compiler does not track; correctness rests on hand-written wait counts
(s_waitcnt vmcnt) before barriers and on the order in which the two halves of
the workgroup (wavefronts 0-3 = group A, 4-7 = group B) read and refill the
stages.  A race there shows up on the GPU only when a DMA is late, so tests
of the outputs cannot be relied on to find it.  This test reads the schedule's
constants out of prefill.hip (stage count, prologue DMA order, loop DMA
offsets, the two wait counts), replays the barrier timeline of both groups
for every loop length up to 14 tiles, and checks that

  * every LDS read of a tile happens after every wavefront (both groups) has
    waited for its own DMA units of that tile before a barrier that precedes
    the read, and
  * no DMA is issued into a stage whose previous tile is still to be read,

and that the checker does find the race the end-of-softmax-half wait closes.
"""
import os
import re

import pytest

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "kv_cache_attention_msa_amd", "csrc", "prefill.hip")


def schedule_constants():
    src = open(SRC).read()
    stages = int(re.search(r"constexpr int kStages = (\d+);", src).group(1))
    waves = int(re.search(r"static constexpr int WAVES = (\d+);", src).group(1))
    upw = 16 // waves  # DMA units of a 16-unit tile per wavefront = DMAs per issue call
    w_older = int(re.search(r"auto wait_older = \[\] \{ asm volatile\(\"s_waitcnt vmcnt\((\d+)\)", src).group(1))
    w_last = int(re.search(r"auto wait_last = \[\] \{ asm volatile\(\"s_waitcnt vmcnt\((\d+)\)", src).group(1))
    pro = src[src.index("const bool grp_b = w >= 4;"):src.index("f32x16_t sc[2];")]
    prologue = [(kind.upper(), int(t)) for kind, t in re.findall(r"issue_(k|v)\((\d+)\);", pro)]
    loop = src[src.index("for (int k = 0; k < n_eff; ++k) {"):]
    dk = int(re.search(r"issue_k\(k \+ (\d+)\);", loop).group(1))
    dv = int(re.search(r"issue_v\(k \+ (\d+)\);", loop).group(1))
    # the loop body of the kept schedule: DMAs, matrix half, wait_older,
    # barrier, softmax half, wait_last, barrier
    body = loop[:loop.index("// A ends one half-step earlier")]
    order = re.findall(r"issue_k|mphase\(|wait_older\(\)|wait_last\(\)|softmax\(", body)
    assert order == ["issue_k", "mphase(", "wait_older()", "softmax(", "wait_last()"], order
    return dict(stages=stages, upw=upw, w_mid=w_older, w_end=w_last, prologue=prologue,
                dk=dk, dv=dv, w_pro=w_older)


class Group:
    """One half of the workgroup: its DMAs in issue order and how many of
    them it has waited for."""

    def __init__(self, upw):
        self.upw = upw
        self.issued = []   # (kind, tile) per DMA instruction
        self.landed = 0    # the first `landed` DMAs are complete

    def issue(self, kind, tile):
        self.issued += [(kind, tile)] * self.upw

    def wait(self, outstanding):
        self.landed = max(self.landed, len(self.issued) - outstanding)


def replay(c, n, w_end=None):
    """Replay the kernel's timeline for n tiles; return a list of violations."""
    w_end = c["w_end"] if w_end is None else w_end
    ns, upw = c["stages"], c["upw"]
    A, B = Group(upw), Group(upw)
    bad = []
    # epochs between barriers: (reads, issues) per group; a snapshot of what
    # both groups had waited for is taken at every barrier
    snap = None

    def barrier():
        nonlocal snap
        snap = ({"A": A.landed, "B": B.landed}, list(A.issued), list(B.issued))

    def check_read(epoch, kind, tile):
        landed, ia, ib = snap
        for name, issued in (("A", ia), ("B", ib)):
            idx = [i for i, d in enumerate(issued) if d == (kind, tile)]
            if len(idx) != upw or max(idx) >= landed[name]:
                bad.append(f"n={n} epoch {epoch}: {kind}({tile}) read before group {name}'s DMAs landed")

    reads = {}  # epoch -> list of (kind, tile)
    issues = {}  # epoch -> list of (kind, tile)

    # prologue: both groups issue, wait, barrier 0
    for g in (A, B):
        for kind, t in c["prologue"]:
            g.issue(kind, t)
        g.wait(c["w_pro"])
    barrier()
    epoch = 1
    # epoch 1: QK(0) by all; A: softmax(0) + wait_last; B: nothing
    reads.setdefault(epoch, []).append(("K", 0))
    reads[epoch].append(("V", 0))
    for kind, t in reads[epoch]:
        check_read(epoch, kind, t)
    A.wait(w_end)
    barrier()
    epoch = 2
    # from here epoch 2+2k: A issue(k) + matrix half k, B softmax(k);
    #            epoch 3+2k: A softmax(k+1), B issue(k) + matrix half k
    for k in range(n):
        # --- epoch 2+2k
        e = 2 + 2 * k
        A.issue("K", k + c["dk"])
        A.issue("V", k + c["dv"])
        issues.setdefault(e, []).extend([("K", k + c["dk"]), ("V", k + c["dv"])])
        r = [("K", k + 1), ("V", k)]       # A: QK(k+1), PV(k)
        r.append(("V", k))                 # B: softmax(k) reads V(k) ahead
        reads.setdefault(e, []).extend(r)
        for kind, t in r:
            check_read(e, kind, t)
        A.wait(c["w_mid"])
        B.wait(w_end)                      # B's softmax(k) half ends with wait_last
        barrier()
        # --- epoch 3+2k
        e = 3 + 2 * k
        B.issue("K", k + c["dk"])
        B.issue("V", k + c["dv"])
        issues.setdefault(e, []).extend([("K", k + c["dk"]), ("V", k + c["dv"])])
        r = [("K", k + 1), ("V", k)]       # B: QK(k+1), PV(k)
        if k + 1 < n:
            r.append(("V", k + 1))         # A: softmax(k+1) reads V(k+1) ahead
        reads.setdefault(e, []).extend(r)
        for kind, t in r:
            check_read(e, kind, t)
        A.wait(w_end)
        B.wait(c["w_mid"])
        barrier()
    # B's last softmax-less half-step: no reads
    # overwrite safety: a DMA of tile X into stage X % ns in epoch e needs no
    # read of tile X - ns in epoch e or later
    last_read = {}
    for e, rs in reads.items():
        for kind, t in rs:
            last_read[(kind, t)] = max(last_read.get((kind, t), -1), e)
    for e, iss in issues.items():
        for kind, t in iss:
            old = (kind, t - ns)
            if old[1] >= 0 and last_read.get(old, -1) >= e:
                bad.append(f"n={n} epoch {e}: DMA of {kind}({t}) overwrites {kind}({t - ns}), "
                           f"still read in epoch {last_read[old]}")
    # the prologue's DMAs (epoch 0) must not overwrite anything read later
    seen = set()
    for kind, t in c["prologue"]:
        for kk, tt in seen:
            if kk == kind and tt % ns == t % ns and tt != t:
                bad.append(f"prologue: {kind}({t}) and {kind}({tt}) share a stage")
        seen.add((kind, t))
    return bad


def test_schedule_constants_parse():
    c = schedule_constants()
    assert c["stages"] >= 3 and c["upw"] >= 1
    assert c["prologue"][0] == ("K", 0)
    assert c["w_end"] < c["w_mid"]


@pytest.mark.parametrize("n", range(1, 15))
def test_every_read_follows_all_dma_waits_and_no_stage_is_overwritten_early(n):
    c = schedule_constants()
    assert replay(c, n) == []


def test_checker_finds_the_race_of_a_loose_end_of_softmax_wait():
    # with the softmax half ending on the looser wait (all but the last two
    # iterations), group A's early read of V(k+1) can run ahead of group B's
    # DMA units of that tile
    c = schedule_constants()
    bad = replay(c, 8, w_end=c["w_mid"])
    assert any("V(" in b and "group B" in b for b in bad), bad
