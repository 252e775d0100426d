"""The library's host side under AddressSanitizer and UndefinedBehaviorSanitizer.

pool.cpp and kvs_mask.cpp (validation, page planning, the page allocator,
staging, the eviction's lazy page tables) are built for the CPU with clang++
and the sanitizers, against tests/host_check/hip_shim.cpp: stand-ins for the
HIP calls and CPU versions of the launches whose results the host reads back
(no GPU code is built).  tests/host_check/driver.cpp interprets operations
over the C ABI; random operation sequences are generated here, every result
line is predicted from the oracle (page plans: "Leyline", sections 2.1-2.3;
eviction: "KV-streams", "how it works"; the block store: "Leyline", section
3), and a sanitizer report ends the driver with a non-zero status.

Physical page numbers are compared exactly: the library and the oracle both
take the lowest free pages, in batch order."""

import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from oracle import leyline_oracle as O  # noqa: E402

CSRC = os.path.join(ROOT, "mla_paged_cache_amd", "csrc")
HC = os.path.join(ROOT, "tests", "host_check")
CLANG = "/opt/rocm/llvm/bin/clang++"
FLAGS = ["-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{ROOT}/include",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
OK, EINVAL, ERANGE, ENOMEM, EUNSUPPORTED = 0, -1, -2, -3, -4
CODE = {O.InvalidRequest: EINVAL, O.OutOfRange: ERANGE, O.OutOfPages: ENOMEM, O.Unsupported: EUNSUPPORTED}


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not (os.path.exists(CLANG) and os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h")):
        pytest.skip("ROCm clang++ and HIP headers are needed for the host build")
    d = tmp_path_factory.mktemp("host_check")
    srcs = [os.path.join(CSRC, "pool.cpp"), os.path.join(CSRC, "kvs_mask.cpp"),
            os.path.join(HC, "hip_shim.cpp"), os.path.join(HC, "driver.cpp")]
    procs, objs = [], []
    for s in srcs:
        o = str(d / (os.path.basename(s) + ".o"))
        objs.append(o)
        procs.append(subprocess.Popen([CLANG, "-x", "c++", *FLAGS, "-c", s, "-o", o],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p, s in zip(procs, srcs):
        out, _ = p.communicate()
        assert p.returncode == 0, f"{s}:\n{out}"
    exe = str(d / "driver")
    r = subprocess.run([CLANG, "-fsanitize=address,undefined", *objs, "-o", exe, "-lpthread"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def run(exe, lines):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=87")
    r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, env=env,
                       timeout=300)
    assert r.returncode == 0, f"driver exit {r.returncode}\n{r.stderr[-6000:]}"
    assert "runtime error" not in r.stderr, r.stderr[-6000:]
    return r.stdout.splitlines()


class Model:
    """Generates operations and the driver's expected output lines from the
    oracle's bookkeeping (rows are not modelled)."""

    def __init__(self, kind, P, seed, layers=2, max_seqs=5, max_len=700):
        self.kind, self.P, self.L = kind, P, layers
        self.max_seqs, self.max_len = max_seqs, max_len
        self.num_pages = {1: 1600, 4: 400, 16: 100}[P]
        self.max_pages = -(-max_len * 2 // P)
        self.st = O.CacheState.empty(layers, self.num_pages, P, self.max_pages, with_rows=False)
        self.rng = np.random.default_rng(seed)
        self.reuse = True       # the pool's page-reuse setting
        self.ops, self.expect = [], []
        self.emit(f"pool {kind} {layers} {P} {self.num_pages} {max_seqs} {self.max_pages}", "pool 0")

    def emit(self, op, *expect):
        self.ops.append(op)
        self.expect.append(list(expect))

    def live(self):
        return sorted(self.st.tables)

    def books(self):
        out = []
        for s in range(self.max_seqs):
            if s in self.st.tables:
                t = self.st.tables[s]
                out.append(" ".join(map(str, ["seq", s, 0, self.st.lengths[s], self.st.next_pos[s], len(t), *t])))
            else:
                out.append(f"seq {s} {EINVAL}")
        out.append(f"free 0 {len(self.st.free)}")
        self.emit("books", *out)

    # -- operations
    def alloc(self, n=None):
        n = int(self.rng.integers(0, self.max_len)) if n is None else n
        need = -(-n // self.P)
        ids = [s for s in range(self.max_seqs) if s not in self.st.tables]
        if need > self.max_pages:
            self.emit(f"alloc {n}", f"alloc {ERANGE} -1")
        elif not ids or need > len(self.st.free):
            self.emit(f"alloc {n}", f"alloc {ENOMEM} -1")
        else:
            self.st.set_pages(ids[0], sorted(self.st.free)[:need], n)
            self.emit(f"alloc {n}", f"alloc 0 {ids[0]}")

    def free(self):
        if self.rng.random() < 0.1:
            dead = [s for s in range(self.max_seqs + 2) if s not in self.st.tables]
            self.emit(f"free {dead[0]}", f"free {EINVAL}")
            return
        if not self.st.tables:
            return
        s = int(self.rng.choice(self.live()))
        self.st.free |= set(self.st.tables.pop(s))
        del self.st.lengths[s], self.st.next_pos[s]
        self.emit(f"free {s}", "free 0")

    def set_pages(self):
        if not self.st.tables:
            return
        s = int(self.rng.choice(self.live()))
        n = int(self.rng.integers(0, self.max_len))
        need = -(-n // self.P)
        pool = list(self.st.tables[s]) + sorted(self.st.free)
        if need > len(pool):
            return
        pages = [int(x) for x in self.rng.permutation(pool)[:need]]
        others = [p for t, v in self.st.tables.items() if t != s for p in v]
        if others and need and self.rng.random() < 0.15:
            pages[0] = int(self.rng.choice(others))       # a page another sequence holds
            self.emit(f"set {s} {n} {need} " + " ".join(map(str, pages)), f"set {EINVAL}")
            return
        self.st.set_pages(s, pages, n)
        self.emit(f"set {s} {n} {need} " + " ".join(map(str, pages)), "set 0")

    def splice(self):
        if not self.st.tables:
            return
        k = int(self.rng.integers(1, min(3, len(self.st.tables)) + 1))
        seqs = [int(x) for x in self.rng.choice(self.live(), size=k, replace=False)]
        ds, toks = [], []
        for s in seqs:
            n = self.st.lengths[s]
            s0 = int(self.rng.integers(0, n + 1))
            s1 = int(self.rng.integers(s0, n + 1))
            u = self.rng.random()
            mode = O.FORGET if u < 0.12 else (int(self.rng.integers(2, 5)) if u < 0.15 else O.AMORTIZE)
            r = int(self.rng.integers(0, 2 * self.P + 4)) if mode == O.AMORTIZE else 0
            if self.rng.random() < 0.03:
                s1 = n + 1                                 # span past the end
            ds.append(O.Directive(s, s0, s1, r, np.zeros(1) if r else None, mode))
            toks.append(f"{s} {mode} {s0} {s1} {r}")
        if self.rng.random() < 0.05:
            ds.append(ds[0])                               # a sequence twice in one batch
            toks.append(toks[0])
        op = f"splice {int(self.rng.integers(0, 2))} {int(self.rng.integers(0, 2))} {len(ds)} " + " ".join(toks)
        try:
            new, plans = O.splice(self.st, ds, reuse_pages=self.reuse)
        except O.OracleError as e:
            self.emit(op, f"splice {CODE[type(e)]} 0 0")
            return
        self.emit(op, f"splice 0 {self.fresh(plans)} {self.freed(plans, [d.seq for d in ds])}")
        self.st = new

    def fresh(self, plans):
        return sum(int(np.sum(np.asarray(p) < 0)) for p in plans)

    def freed(self, plans, seqs):
        n = 0
        for p, s in zip(plans, seqs):
            kept = {int(x) for x in p if x >= 0}
            n += sum(1 for q in range(len(self.st.tables[s])) if q not in kept)
        return n

    def evict(self, masks_for=None):
        if not self.st.tables:
            return
        if masks_for is None:
            k = int(self.rng.integers(1, min(3, len(self.st.tables)) + 1))
            seqs = [int(x) for x in self.rng.choice(self.live(), size=k, replace=False)]
            masks = []
            for s in seqs:
                n = self.st.lengths[s]
                kind = int(self.rng.integers(0, 5))
                if kind == 0:
                    m = np.ones(n, np.uint8)
                elif kind == 1:
                    m = np.zeros(n, np.uint8)
                elif kind == 2:
                    m = (self.rng.random(n) < self.rng.random()).astype(np.uint8)
                elif kind == 3:
                    m = np.repeat(self.rng.integers(0, 2, size=-(-n // self.P)), self.P)[:n].astype(np.uint8)
                else:
                    m = np.repeat(self.rng.integers(0, 2, size=-(-n // 7)), 7)[:n].astype(np.uint8)
                masks.append(m)
        else:
            seqs, masks = masks_for
        toks = [f"{s} {''.join(map(str, m)) or '-'}" for s, m in zip(seqs, masks)]
        op = f"evict {len(seqs)} " + " ".join(toks)
        try:
            new, plans = O.evict(self.st, seqs, masks, reuse_pages=self.reuse)
        except O.OracleError as e:
            self.emit(op, f"evict {CODE[type(e)]} 0 0")
            return
        self.emit(op, f"evict 0 {self.fresh(plans)} {self.freed(plans, seqs)}")
        self.st = new

    def set_reuse(self):
        """Page reuse on or off (off is refused at page size 1)."""
        on = int(self.rng.random() < 0.6)
        if not on and self.P == 1:
            self.emit("reuse 0", f"reuse {EUNSUPPORTED}")
            return
        self.reuse = bool(on)
        self.emit(f"reuse {on}", "reuse 0")

    def set_limit(self):
        """Work-items per row-kernel dispatch: the packet's own limit, or one
        low enough that every moving call runs as many dispatches (the books
        must not change)."""
        items = int(self.rng.choice([0, 1024, 5000]))
        self.emit(f"limit {items}", "limit 0")

    def reindex(self):
        cand = [s for s in self.live() if self.st.lengths[s] > 0]
        if not cand:
            return
        s = int(self.rng.choice(cand))
        n = self.st.lengths[s]
        n_pages = -(-n // self.P)
        keep = sorted(int(x) for x in np.flatnonzero(self.rng.random(n_pages) < 0.6))
        if self.rng.random() < 0.1 and len(keep) >= 2:
            keep[0], keep[1] = keep[1], keep[0]            # not increasing
        op = f"reindex {s} {len(keep)} " + " ".join(map(str, keep))
        try:
            self.st = O.ptable_reindex(self.st, s, keep)
            self.emit(op, "reindex 0")
        except O.OracleError as e:
            self.emit(op, f"reindex {CODE[type(e)]}")

    def rope(self):
        if not self.st.tables:
            return
        s = int(self.rng.choice(self.live()))
        n = self.st.lengths[s]
        r0 = int(self.rng.integers(0, n + 1))
        cnt = int(self.rng.integers(0, n - r0 + 1))
        if self.rng.random() < 0.1:
            cnt = n - r0 + 1                               # one row past the end
        ok = r0 + cnt <= n
        self.emit(f"rope {s} {r0} {cnt} {int(self.rng.integers(0, 2))}", f"rope {OK if ok else EINVAL}")

    def lengths(self):
        live = self.live()
        if not live:
            return
        seqs = [int(x) for x in self.rng.choice(live, size=min(3, len(live)), replace=False)]
        self.emit(f"lengths {len(seqs)} " + " ".join(map(str, seqs)),
                  "lengths 0 " + " ".join(str(self.st.lengths[s]) for s in seqs))

    def pressure(self):
        """Fill the pool with two long sequences, then evict so that the
        fresh pages the masks need exceed the free ones (refused, nothing
        changed) and then fit."""
        for s in self.live():
            self.st.free |= set(self.st.tables.pop(s))
            del self.st.lengths[s], self.st.next_pos[s]
            self.emit(f"free {s}", "free 0")
        cap = self.num_pages * self.P
        big = min(self.max_len, cap // 2 - 2 * self.P)
        self.alloc(big)
        self.alloc(big)
        self.alloc(len(self.st.free) * self.P + 1)         # one row more than the free pages hold
        self.books()
        if self.P > 1:
            # every new page is fresh: drop row 0 of each sequence
            m = np.ones(big, np.uint8)
            m[0] = 0
            self.evict(([0, 1], [m, m.copy()]))
            self.books()
        self.evict(([0], [np.repeat(self.rng.integers(0, 2, size=-(-big // self.P)), self.P)[:big].astype(np.uint8)]))
        self.books()


@pytest.mark.parametrize("kind,P", [("mla", 1), ("mla", 4), ("mla", 16), ("gqa", 1), ("gqa", 4)])
def test_random_operations_under_sanitizers(driver, kind, P):
    m = Model(kind, P, seed=900 + P + (50 if kind == "gqa" else 0))
    ops = [m.alloc, m.alloc, m.free, m.set_pages, m.splice, m.splice, m.splice, m.evict, m.evict, m.evict,
           m.reindex, m.rope, m.lengths, m.set_reuse, m.set_limit]
    for i in range(260):
        ops[int(m.rng.integers(0, len(ops)))]()
        m.books()
        if i == 130:
            m.pressure()
    m.emit("misc", f"misc 0 0 0 {EINVAL} {EINVAL} 1 LL_ENOMEM")
    got = run(driver, m.ops)
    want = [line for e in m.expect for line in e]
    assert len(got) == len(want), (len(got), len(want))
    k = 0
    for op, exp in zip(m.ops, m.expect):
        for line in exp:
            assert got[k] == line, f"operation {op!r}: got {got[k]!r}, expected {line!r}"
            k += 1


def kvs_line(n_pad, logs):
    parts = [f"kvs {n_pad} {len(logs)}"]
    for n_tokens, events in logs:
        parts.append(f"{n_tokens} {len(events)} " + " ".join(f"{t} {m}" for t, m in events))
    return " ".join(parts)


def test_kvs_host_validation_under_sanitizers(driver):
    """kvs_death_times validates the logs on the host ("KV-streams", "how it
    works": event times increase inside (0, T], an event's mask covers at
    most the tokens generated by then); block and dense masks check their
    shapes.  Valid and invalid requests alike must run clean."""
    rng = np.random.default_rng(5)
    ops, want = [], []
    for _ in range(60):
        n_pad = int(rng.integers(1, 3000))
        logs = []
        for _ in range(int(rng.integers(1, 4))):
            n_tokens = int(rng.integers(0, n_pad + 1))
            times = sorted(set(int(x) for x in rng.integers(1, n_tokens + 1, size=int(rng.integers(0, 6))))) \
                if n_tokens else []
            logs.append((n_tokens, [(t, int(rng.integers(0, t + 1))) for t in times]))
        ops.append(kvs_line(n_pad, logs))
        want.append("kvs 0")
        bad = int(rng.integers(0, 5))
        if bad == 0:
            logs[0] = (n_pad + 1, [])                       # longer than n_pad
        elif bad == 1:
            logs[0] = (logs[0][0] + 2, [(2, 0), (1, 0)])    # times decrease
        elif bad == 2:
            logs[0] = (logs[0][0] + 1, [(0, 0)])            # time 0
        elif bad == 3:
            logs[0] = (logs[0][0] + 3, [(3, 4)])            # mask longer than the tokens so far
        else:
            logs[0] = (logs[0][0] + 1, [(logs[0][0] + 2, 0)])  # after the last token
        ops.append(kvs_line(n_pad if bad == 0 else max(n_pad, logs[0][0]), logs))
        want.append(f"kvs {EINVAL}")
    ops.append(kvs_line(0, [(0, [])]))
    want.append(f"kvs {EINVAL}")
    # n_pad beyond the LDS list: the context's list scratch, grown, then reused
    for n_pad, n in [(50000, 1), (60000, 2), (50000, 2), (1000, 1), (70000, 1)]:
        ops.append(kvs_line(n_pad, [(n_pad - 5, [(100, 50), (n_pad - 10, min(3000, n_pad - 10))])] * n))
        want.append("kvs 0")
    for n, n_pad, bq, bk, exp in [(2, 256, 16, 32, "0 0"), (1, 1024, 1024, 16, "0 0"), (3, 100, 64, 64, f"0 {EINVAL}"),
                                  (2, 256, 8, 32, f"{EINVAL} 0"), (2, 256, 48, 32, f"{EINVAL} 0"),
                                  (2, 384, 2048, 16, f"{EINVAL} 0")]:
        ops.append(f"kvsmask {n} {n_pad} {bq} {bk}")
        want.append(f"kvsmask {exp}")
    assert run(driver, ops) == want
