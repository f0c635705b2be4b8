"""The library's index-producing kernels built for the CPU and checked
against the oracle, on every `pytest` run (no GPU needed).

``tests/host/host_kernels.cpp`` compiles bucket.hip and cache.hip unchanged
against a stand-in HIP runtime (``tests/host/hip/hip_runtime.h``: the
threads of a workgroup as fibers, barriers and wave operations -- shuffles,
ballot, DPP row moves, lane reads -- as rendezvous) with AddressSanitizer
and UBSan, and gives every buffer exactly the size the library's context
gives it.  A kernel index past the end of a work list, perm, offsets array,
activation record, miss list or slot table therefore aborts the harness and
fails the test; so does a barrier or wave operation that some thread of a
block skips.

Checked here, on the same seeded inputs as the oracle:
* bucketing (both the one-workgroup path, n <= 1,024 pairs, and the
  histogram/scan/scatter path) -- offsets and perm equal to ``oracle.bucket``,
  ids outside [0, E) ignored, nothing written past the valid pairs;
* the work list the FFN kernels walk, equal to its definition (per expert
  ceil(count / m) entries of <= m pairs, ascending expert, then the shared
  expert's T tokens), at the decode (m = 4) and prefill (m = 128) entry sizes;
* the decode x record built in the same launch, equal to its definition
  (values in MFMA step order, divided by the code-slot factor, split into
  fp16 hi and lo halves), ragged d_model included;
* moe_bucket_noalloc on both paths (its static scratch on the large one);
* cache resolve with the zero-copy miss fill: slot_of_pair, the miss list
  and counts call by call, the final table and stamps against
  ``oracle.LRUCache``, every occupied slot holding its identity's blob; a
  call that cannot pin its working set; the resident (identity) map; ids
  outside [0, E).
"""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CLANG = "/opt/rocm/llvm/bin/clang++"
POISON = np.int32(-1515870811)  # 0xa5a5a5a5: the fill of every output buffer before the launch


@pytest.fixture(scope="session")
def exe(tmp_path_factory):
    if not os.path.exists(CLANG):
        pytest.skip(f"{CLANG} not found (the host build needs ROCm's clang and its sanitizer runtimes)")
    out = str(tmp_path_factory.mktemp("host_kernels") / "host_kernels")
    cmd = [CLANG, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-rtlib=compiler-rt", "-unwindlib=libgcc",
           "-I", os.path.join(HERE, "host"), "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "host", "host_kernels.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return out


def _run(exe, tmp_path, args, data):
    fin, fout = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    np.concatenate([np.asarray(a).reshape(-1).view(np.int32) for a in data]).tofile(fin)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", HOSTK_SEED="7")
    r = subprocess.run([exe] + [str(a) for a in args] + [fin, fout], capture_output=True, text=True, env=env,
                       timeout=600)
    errs = "\n".join(l for l in r.stderr.splitlines() if "doesn't fully support makecontext" not in l)
    assert r.returncode == 0 and "ERROR" not in errs and "runtime error" not in errs, errs[-6000:]
    return np.fromfile(fout, dtype=np.int32)


class _Reader:
    def __init__(self, a):
        self.a, self.p = a, 0

    def take(self, n, dtype=np.int32):
        w = n * np.dtype(dtype).itemsize // 4
        v = self.a[self.p:self.p + w].view(dtype)
        self.p += w
        assert v.size == n, "short harness output"
        return v

    def done(self):
        assert self.p == self.a.size


# ---------------------------------------------------------------------------
# expected values
# ---------------------------------------------------------------------------

def _bucket_expected(idx, E):
    """oracle.bucket over the valid pairs: ids outside [0, E) go to a virtual
    expert E, which sorts last and is then dropped."""
    flat = np.asarray(idx).reshape(-1).astype(np.int64)
    v = np.where((flat >= 0) & (flat < E), flat, E)
    counts, offsets, perm = oracle.bucket(v, E + 1)
    return counts[:E], offsets[:E + 1], perm[:offsets[E]]


def _work_expected(counts, offsets, T, m):
    ents = []
    for e, c in enumerate(counts):
        for i in range(-(-int(c) // m)):
            ents.append((e, int(offsets[e]) + i * m, min(m, int(c) - i * m), 0))
    routed = len(ents)
    for i in range(-(-T // m)):
        ents.append((-1, i * m, min(m, T - i * m), 0))
    return np.array(ents, dtype=np.int32).reshape(-1, 4), routed


def _xrec_expected(x, nsb):
    """The decode x record by its definition: per token, superblock S and
    MFMA step t, 8 hi halves then 8 lo halves; half 2q + h holds column
    c + 5h of code pair p = 4t + q, c = 160 S + 10 (p // 5) + p % 5, divided
    by f = 8^((p % 5) % 3); hi = fp16(v), lo = fp16(v - hi); columns past
    d_model hold zero; one extra all-zero row."""
    T, d = x.shape
    rec = np.zeros((T + 1, nsb, 20, 2, 8), dtype=np.uint16)
    for S in range(nsb):
        for t in range(20):
            for q in range(4):
                p = 4 * t + q
                for h in range(2):
                    col = 160 * S + 10 * (p // 5) + p % 5 + 5 * h
                    f = np.float32(8.0 ** ((p % 5) % 3))
                    v = (x[:, col] / f).astype(np.float32) if col < d else np.zeros(T, np.float32)
                    hi = v.astype(np.float16)
                    lo = (v - hi.astype(np.float32)).astype(np.float16)
                    rec[:T, S, t, 0, 2 * q + h] = hi.view(np.uint16)
                    rec[:T, S, t, 1, 2 * q + h] = lo.view(np.uint16)
    return rec.reshape(T + 1, -1)


def _routing(rng, T, k, E, zipf=0.0):
    p = 1.0 / np.arange(1, E + 1) ** zipf
    p /= p.sum()
    return np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


# ---------------------------------------------------------------------------
# bucketing and work list
# ---------------------------------------------------------------------------

BUCKET_CASES = [
    # (E, T, k, entry_m, d_model, what)
    (512, 15, 10, 4, 320, "decode workload: 150 pairs, x record of 2 superblocks"),
    (512, 1, 10, 4, 224, "one token; ragged d_model (224 = 160 + 64)"),
    (64, 128, 8, 4, 0, "exactly 1,024 pairs, the largest one-workgroup case"),
    (1024, 1, 1, 4, 0, "1,024 experts, one pair"),
    (1, 37, 1, 4, 96, "one expert: every pair in one bucket"),
    (512, 103, 10, 128, 0, "1,030 pairs: the multi-workgroup path, prefill entry size"),
    (512, 1000, 10, 128, 0, "10,000 pairs: 40 chunks, two scan batches"),
    (128, 600, 4, 4, 0, "2,400 pairs at the decode entry size"),
]


@pytest.mark.parametrize("E,T,k,m,d,what", BUCKET_CASES, ids=[c[-1].split(":")[0] for c in BUCKET_CASES])
def test_bucket_and_work_list(exe, tmp_path, E, T, k, m, d, what):
    rng = np.random.default_rng(E * 7 + T)
    idx = _routing(rng, T, k, E, zipf=0.8) if k <= E else None
    data = [idx]
    x = None
    if d:
        x = rng.standard_normal((T, d)).astype(np.float32) * np.float32(3.0)
        data.append(x.view(np.int32))
    out = _Reader(_run(exe, tmp_path, ["bucket", E, T, k, m, 1, d], data))
    counts, offsets, perm = _bucket_expected(idx, E)
    assert np.array_equal(out.take(E + 1), offsets)
    assert np.array_equal(out.take(T * k), perm)
    n_work = out.take(2)
    work, routed = _work_expected(counts, offsets, T, m)
    assert n_work.tolist() == [len(work), routed]
    assert np.array_equal(out.take(len(work) * 4).reshape(-1, 4), work)
    if m == 4:  # the decode path's second list: entries of up to 8 pairs
        work8, routed8 = _work_expected(counts, offsets, T, 8)
        assert out.take(2).tolist() == [len(work8), routed8]
        assert np.array_equal(out.take(len(work8) * 4).reshape(-1, 4), work8)
    if d:
        nsb = -(-d // 160)
        got = out.take((T + 1) * nsb * 320, np.uint16).reshape(T + 1, -1)
        assert np.array_equal(got, _xrec_expected(x, nsb))
    out.done()


@pytest.mark.parametrize("T,k,E", [(9, 4, 16), (300, 8, 64)], ids=["one_workgroup", "multi_workgroup"])
def test_bucket_ignores_ids_outside_range(exe, tmp_path, T, k, E):
    rng = np.random.default_rng(5)
    idx = rng.integers(-3, E + 3, size=(T, k)).astype(np.int32)
    idx[0, 0], idx[-1, -1] = -1, E  # at least one of each kind
    out = _Reader(_run(exe, tmp_path, ["bucket", E, T, k, 4, 1, 0], [idx]))
    counts, offsets, perm = _bucket_expected(idx, E)
    assert np.array_equal(out.take(E + 1), offsets)
    got = out.take(T * k)
    nv = int(offsets[E])
    assert np.array_equal(got[:nv], perm) and np.all(got[nv:] == POISON)  # nothing past the valid pairs
    n_work = out.take(2)
    work, routed = _work_expected(counts, offsets, T, 4)
    assert n_work.tolist() == [len(work), routed]
    assert np.array_equal(out.take(len(work) * 4).reshape(-1, 4), work)
    work8, routed8 = _work_expected(counts, offsets, T, 8)
    assert out.take(2).tolist() == [len(work8), routed8]
    assert np.array_equal(out.take(len(work8) * 4).reshape(-1, 4), work8)
    out.done()


@pytest.mark.parametrize("T,k,E", [(15, 10, 512), (2000, 10, 512), (13107, 10, 1024)],
                         ids=["one_workgroup", "scratch_path", "max_pairs"])
def test_noalloc_bucket(exe, tmp_path, T, k, E):
    rng = np.random.default_rng(T)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)  # repeats allowed: the bucketing does not care
    out = _Reader(_run(exe, tmp_path, ["noalloc", E, T, k], [idx]))
    assert out.take(1)[0] == 0
    _counts, offsets, perm = _bucket_expected(idx, E)
    assert np.array_equal(out.take(E + 1), offsets)
    assert np.array_equal(out.take(T * k), perm)
    out.done()


# ---------------------------------------------------------------------------
# cache resolve and miss fill
# ---------------------------------------------------------------------------

def _resolve(exe, tmp_path, L, E, S, T, k, calls, fill=1, resident=0, dm=64, dff=64):
    recs = []
    for layer, idx in calls:
        recs.append(np.int32(layer).reshape(1))
        recs.append(idx.astype(np.int32))
    out = _Reader(_run(exe, tmp_path, ["resolve", L, E, S, T, k, len(calls), fill, resident, dm, dff], recs))
    per_call = [(out.take(3).copy(), out.take(T * k).copy()) for _ in calls]
    stats = out.take(6, np.int64)
    tail = None
    if not resident:
        tail = (out.take(L * E), out.take(S), out.take(S, np.uint32), out.take(1)[0])
    out.done()
    return per_call, stats, tail


def _check_lru(per_call, stats, tail, L, E, S, calls):
    orc = oracle.LRUCache(L, E, S)
    failed = 0
    for (dm, sop), (layer, idx) in zip(per_call, calls):
        flat = idx.reshape(-1)
        valid = (flat >= 0) & (flat < E)
        nuniq = len(np.unique(flat[valid]))
        if nuniq > S:
            with pytest.raises(oracle.CapacityError):
                orc.resolve(layer, flat[valid])
            failed += 1
            assert dm.tolist() == [nuniq, 0, 1] and np.all(sop == -1)
            continue
        so, misses = orc.resolve(layer, flat[valid])
        want = np.full(flat.size, -1, np.int32)
        want[valid] = so
        assert dm.tolist() == [nuniq, len(misses), 0]
        assert np.array_equal(sop, want)
    slot_of, id_of, stamp, bad_blobs = tail
    assert slot_of.tolist() == orc.slot_of
    assert id_of.tolist() == orc.id_of.tolist() and stamp.tolist() == orc.stamp.tolist()
    assert bad_blobs == 0  # every occupied slot holds its identity's blob
    assert stats.tolist() == [orc.lookups, orc.hits, orc.misses, len(calls) - failed, failed, orc.clock]
    return orc


def test_resolve_lru_with_fill(exe, tmp_path):
    L, E, S, T, k = 4, 64, 40, 3, 4
    rng = np.random.default_rng(11)
    calls = [(c % L, _routing(rng, T, k, E, zipf=1.1)) for c in range(36)]
    per_call, stats, tail = _resolve(exe, tmp_path, L, E, S, T, k, calls)
    orc = _check_lru(per_call, stats, tail, L, E, S, calls)
    assert orc.hits > 0 and orc.misses > S  # the table filled and evicted


def test_resolve_with_the_fill_in_the_bucketing_launch(exe, tmp_path):
    # no fill kernel: the bucketing launch of a capped decode layer copies the
    # misses in its spare workgroups; the same table and slot contents as with
    # the fill kernel, failed calls and ids outside the range included
    L, E, S, T, k = 3, 48, 7, 2, 4
    rng = np.random.default_rng(15)
    calls = []
    for c in range(40):
        if c % 9 == 8:  # 8 distinct ids > 7 slots: the call fails and changes nothing
            idx = rng.permutation(E)[:T * k].reshape(T, k)
        else:
            idx = _routing(rng, T, k, E, zipf=1.1)
            idx[rng.random((T, k)) < 0.1] = rng.choice([-1, E])
        calls.append((c % L, idx.astype(np.int32)))
    per_call, stats, tail = _resolve(exe, tmp_path, L, E, S, T, k, calls, fill=2)
    orc = _check_lru(per_call, stats, tail, L, E, S, calls)
    assert orc.misses > S and orc.hits > 0 and stats[4] >= 4


def test_resolve_capacity_failure_and_ids_outside_range(exe, tmp_path):
    L, E, S, T, k = 2, 32, 8, 3, 4
    rng = np.random.default_rng(12)
    calls = []
    for c in range(24):
        if c % 6 == 5:  # 12 distinct ids > 8 slots: the call fails and changes nothing
            idx = rng.permutation(E)[:T * k].reshape(T, k).astype(np.int32)
        else:
            idx = rng.choice(E // 4, size=(T, k)).astype(np.int32)  # repeats: few distinct ids
            idx[rng.random((T, k)) < 0.2] = rng.choice([-1, E, E + 7])
        calls.append((c % L, idx))
    per_call, stats, tail = _resolve(exe, tmp_path, L, E, S, T, k, calls)
    orc = _check_lru(per_call, stats, tail, L, E, S, calls)
    assert stats[4] == 4 and orc.misses > 0


def test_resolve_without_fill_leaves_pairs_on_failure(exe, tmp_path):
    # the host-copy path: on a failed call the kernel writes no slot (the host reads the error)
    L, E, S, T, k = 1, 16, 3, 2, 2
    calls = [(0, np.array([[0, 1], [1, 2]], np.int32)), (0, np.array([[0, 5], [6, 7]], np.int32)),
             (0, np.array([[2, 1], [0, 0]], np.int32))]
    per_call, stats, _tail = _resolve(exe, tmp_path, L, E, S, T, k, calls, fill=0)
    assert per_call[0][0].tolist() == [3, 3, 0] and sorted(per_call[0][1].tolist()) == [0, 1, 1, 2]
    assert per_call[1][0].tolist() == [4, 0, 1] and np.all(per_call[1][1] == POISON)
    assert per_call[2][0].tolist() == [3, 0, 0]
    assert stats.tolist() == [6, 3, 3, 2, 1, 2]


def test_resolve_resident_identity_map(exe, tmp_path):
    L, E, T, k = 3, 64, 5, 6
    rng = np.random.default_rng(13)
    calls = []
    for c in range(6):
        idx = _routing(rng, T, k, E)
        idx[0, 0] = -2 if c % 2 else E
        calls.append((c % L, idx))
    per_call, stats, _ = _resolve(exe, tmp_path, L, E, L * E, T, k, calls, resident=1)
    lookups = 0
    for (dm, sop), (layer, idx) in zip(per_call, calls):
        flat = idx.reshape(-1)
        valid = (flat >= 0) & (flat < E)
        nuniq = len(np.unique(flat[valid]))
        lookups += nuniq
        assert dm.tolist() == [nuniq, 0, 0]
        assert np.array_equal(sop, np.where(valid, layer * E + flat, -1))
    assert stats[:5].tolist() == [lookups, lookups, 0, len(calls), 0]


@pytest.mark.parametrize("T", [1, 2])
def test_route_resolve_one_workgroup(exe, tmp_path, T):
    # a capped decode layer of one or two tokens: the router's top-k from the
    # partial logits, token after token, then the resolve, in one workgroup of
    # 1,024 threads -- logits bit for bit (slices summed in order, then the
    # bias, in float32), idx the oracle's top-k of those logits (exact ties
    # included), w its weights, slots and table the oracle LRU's
    L, E, S, k, KS, calls = 3, 512, 40, 10, 8, 10
    rng = np.random.default_rng(20 + T)
    bias = (rng.normal(0.0, 1.0, E) + 2.0 * (np.arange(E) < 24)).astype(np.float32)  # a hot set: hits
    bias[40:52] = bias[40]
    parts = []
    for c in range(calls):
        p = rng.normal(0.0, 0.5, (KS, T, E)).astype(np.float32)
        if c % 4 == 1:  # exact ties among the leaders: twelve experts with equal partials and bias
            p[:, :, 40:52] = 1.5
        parts.append(p)
    recs = [bias.view(np.int32)]
    for c, p in enumerate(parts):
        recs += [np.int32(c % L).reshape(1), p.view(np.int32)]
    out = _Reader(_run(exe, tmp_path, ["route_resolve", L, E, S, T, k, KS, calls], recs))
    orc = oracle.LRUCache(L, E, S)
    for c, p in enumerate(parts):
        logits = out.take(T * E, np.float32).reshape(T, E)
        idx = out.take(T * k).reshape(T, k)
        w = out.take(T * k, np.float32).reshape(T, k)
        dm, sop = out.take(3), out.take(T * k)
        want = np.zeros((T, E), np.float32)
        for q in range(KS):
            want = want + p[q]
        want = want + bias
        assert np.array_equal(logits.view(np.int32), want.view(np.int32)), c
        idx_o, w_o = oracle.topk_from_logits(want.astype(np.float64), k)
        assert np.array_equal(idx, idx_o), (c, idx, idx_o)
        assert np.allclose(w, w_o, rtol=1e-6, atol=1e-7), c
        so, misses = orc.resolve(c % L, idx.reshape(-1))
        assert dm.tolist() == [len(np.unique(idx)), len(misses), 0] and np.array_equal(sop, so.reshape(-1)), c
    stats = out.take(6, np.int64)
    slot_of, id_of, stamp = out.take(L * E), out.take(S), out.take(S, np.uint32)
    out.done()
    assert stats.tolist() == [orc.lookups, orc.hits, orc.misses, calls, 0, orc.clock]
    assert slot_of.tolist() == orc.slot_of and id_of.tolist() == orc.id_of.tolist()
    assert stamp.tolist() == orc.stamp.tolist()
    assert orc.hits > 0 and orc.misses > 0


@pytest.mark.slow
def test_resolve_more_slots_than_threads(exe, tmp_path):
    # 1,100 slots: the victim search strides past the workgroup's 1,024
    # threads; ~1,180 misses fill the table and then evict
    L, E, S, T, k = 3, 512, 1100, 1, 32
    rng = np.random.default_rng(14)
    calls = [(c % L, _routing(rng, T, k, E)) for c in range(70)]
    per_call, stats, tail = _resolve(exe, tmp_path, L, E, S, T, k, calls, fill=1, dm=64, dff=64)
    orc = _check_lru(per_call, stats, tail, L, E, S, calls)
    assert int(np.sum(orc.id_of >= 0)) == S and orc.misses > S


# ---------------------------------------------------------------------------
# the bucketing launch of a resident decode layer, with its lookup count
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 2])
def test_route_bucket_one_or_two_tokens(exe, tmp_path, T):
    # a resident decode layer of one or two tokens: the top-k of each token
    # (from partial logits, exact ties included) and then the bucketing, the
    # work lists, the lookup count and the x record in one launch -- against
    # the oracle's top-k of the launch's own logits and the bucketing of its idx
    E, k, d, KS = 512, 10, 320, 8
    rng = np.random.default_rng(40 + T)
    bias = rng.normal(0.0, 1.0, E).astype(np.float32)
    bias[100:112] = bias[100]
    part = rng.normal(0.0, 0.5, (KS, T, E)).astype(np.float32)
    part[:, :, 100:112] = 1.5  # twelve experts tied at the top
    x = (rng.standard_normal((T, d)) * 2.0).astype(np.float32)
    out = _Reader(_run(exe, tmp_path, ["route_bucket", KS, E, T, k, d], [bias.view(np.int32), part.view(np.int32),
                                                                         x.view(np.int32)]))
    logits = out.take(T * E, np.float32).reshape(T, E)
    want = np.zeros((T, E), np.float32)
    for q in range(KS):
        want = want + part[q]
    want = want + bias
    assert np.array_equal(logits.view(np.int32), want.view(np.int32))
    idx = out.take(T * k).reshape(T, k)
    w = out.take(T * k, np.float32).reshape(T, k)
    idx_o, w_o = oracle.topk_from_logits(want.astype(np.float64), k)
    assert np.array_equal(idx, idx_o) and np.allclose(w, w_o, rtol=1e-6, atol=1e-7)
    assert idx[0].tolist() == list(range(100, 110))  # ties broken by index
    counts, offsets, perm = _bucket_expected(idx, E)
    assert np.array_equal(out.take(E + 1), offsets)
    assert np.array_equal(out.take(T * k), perm)
    work, routed = _work_expected(counts, offsets, T, 4)
    assert out.take(2).tolist() == [len(work), routed]
    assert np.array_equal(out.take(len(work) * 4).reshape(-1, 4), work)
    work8, routed8 = _work_expected(counts, offsets, T, 8)
    assert out.take(2).tolist() == [len(work8), routed8]
    assert np.array_equal(out.take(len(work8) * 4).reshape(-1, 4), work8)
    nsb = -(-d // 160)
    assert np.array_equal(out.take((T + 1) * nsb * 320, np.uint16).reshape(T + 1, -1), _xrec_expected(x, nsb))
    nuniq = len(np.unique(idx))
    assert out.take(3).tolist() == [nuniq, 0, 0]
    assert out.take(6, np.int64).tolist() == [2 * nuniq, 2 * nuniq, 0, 2, 0, 0]
    out.done()


@pytest.mark.parametrize("E,T,k,d", [(512, 15, 10, 2048), (64, 128, 8, 96), (1024, 1, 1, 160)],
                         ids=["decode_workload", "1024_pairs", "1024_experts"])
def test_bucket_lookup(exe, tmp_path, E, T, k, d):
    rng = np.random.default_rng(E + T)
    idx = _routing(rng, T, k, E, zipf=0.8)
    x = (rng.standard_normal((T, d)) * 2.0).astype(np.float32)
    out = _Reader(_run(exe, tmp_path, ["bucket_lookup", E, T, k, d], [idx, x.view(np.int32)]))
    counts, offsets, perm = _bucket_expected(idx, E)
    assert np.array_equal(out.take(E + 1), offsets)
    assert np.array_equal(out.take(T * k), perm)
    n_work = out.take(2)
    work, routed = _work_expected(counts, offsets, T, 4)
    assert n_work.tolist() == [len(work), routed]
    assert np.array_equal(out.take(len(work) * 4).reshape(-1, 4), work)
    work8, routed8 = _work_expected(counts, offsets, T, 8)
    assert out.take(2).tolist() == [len(work8), routed8]
    assert np.array_equal(out.take(len(work8) * 4).reshape(-1, 4), work8)
    nsb = -(-d // 160)
    assert np.array_equal(out.take((T + 1) * nsb * 320, np.uint16).reshape(T + 1, -1), _xrec_expected(x, nsb))
    # what the resolve kernel records for a resident call, twice
    nuniq = len(np.unique(idx))
    assert out.take(3).tolist() == [nuniq, 0, 0]
    assert out.take(6, np.int64).tolist() == [2 * nuniq, 2 * nuniq, 0, 2, 0, 0]
    out.done()
