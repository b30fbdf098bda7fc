"""Seeded parity cases shared by the GPU tests: the same generated inputs go to the HIP path
(through the C ABI binding) and to the CPU oracle. Nothing the oracle consumes comes from the HIP
path; large weight tensors are drawn on the device by the generator's device build, which is
bit-identical to its host build (checked by test_gen_device_bitexact), and the oracle compresses
the host draw of the experts it needs."""
import os
import sys

import numpy as np
import torch

import gen
import oracle as orc
import sparse_precision_grouped_amd as mq

DEV = "cuda"
_cache = {}


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


class OracleWeights:
    """Oracle-compressed weights of one projection, built lazily per expert from the host draw."""

    def __init__(self, cfg, proj, E, N, K):
        self.cfg, self.proj, self.E, self.N, self.K = cfg, proj, E, N, K
        self.packed = np.zeros((E, N, K // 4), np.uint8)
        self.mask = np.zeros((E, N, K // 16), np.uint8)
        self.scale = np.zeros((E, N, K // 32), np.uint8)
        self.gscale = np.zeros(E, np.float32)
        self.done = np.zeros(E, bool)

    def ensure(self, experts):
        for e in sorted(set(int(x) for x in experts)):
            if self.done[e]:
                continue
            w = gen.weights_expert(self.cfg, self.proj, e, self.N, self.K)[None]
            W = orc.compress(w)
            self.packed[e], self.mask[e], self.scale[e], self.gscale[e] = (W["packed"][0], W["mask"][0],
                                                                           W["scale"][0], W["gscale"][0])
            self.done[e] = True
        return self

    def as_dict(self):
        return dict(packed=self.packed, mask=self.mask, scale=self.scale, gscale=self.gscale, E=self.E, N=self.N,
                    K=self.K)


def device_weights(cfg, proj, E, N, K, host_draw):
    """Weights compressed on the device from the generator's draw (host draw copied, or device draw)."""
    if host_draw:
        w = np.stack([gen.weights_expert(cfg, proj, e, N, K) for e in range(E)])
        return mq.moesq_compress_weights(dev(w)), w
    Wd = mq.Weights.empty(E, N, K, DEV)
    buf = torch.empty((min(E, 16), N, K), dtype=torch.float32, device=DEV)
    ws = torch.empty(mq.moesq_workspace_bytes(mq.WS_COMPRESS, 0, 0, 16), dtype=torch.uint8, device=DEV)
    for e0 in range(0, E, 16):
        n = min(16, E - e0)
        for j in range(n):
            gen.gpu_fill_normal(buf[j], cfg.seed, gen.weight_stream(proj, e0 + j), cfg.w_std)
        sub = mq.Weights(Wd.packed[e0:e0 + n], Wd.mask[e0:e0 + n], Wd.scale[e0:e0 + n], Wd.gscale[e0:e0 + n])
        mq.moesq_compress_weights(buf[:n].contiguous() if n < buf.shape[0] else buf, out=sub, workspace=ws,
                                  prepack=False)
    Wd.prepack()
    torch.cuda.synchronize()
    return Wd, None


def single_case(name, proj=0, x_tag=0):
    """A single-projection grouped GEMM case of a named config (proj 1 = the down shape of c3)."""
    key = ("single", name, proj, x_tag)
    if key in _cache:
        return _cache[key]
    cfg = gen.CONFIGS[name]
    E, T, k = cfg.E, cfg.T, cfg.k
    N, K = (cfg.N, cfg.K) if proj == 0 else (cfg.N2, cfg.K2)
    say("building", name, "proj", proj, "E N K T k =", E, N, K, T, k)
    small = E * N * K <= 512 * 1024 * 1024
    Wd, w = device_weights(cfg, proj, E, N, K, host_draw=small)
    Wo = OracleWeights(cfg, proj, E, N, K)
    if w is not None:
        W = orc.compress(w)
        Wo.packed, Wo.mask, Wo.scale, Wo.gscale = W["packed"], W["mask"], W["scale"], W["gscale"]
        Wo.done[:] = True
    x = gen.activations(cfg, x_tag, T, K)
    ids, wts = gen.routing(cfg)
    R = orc.route(ids, E)
    ga = np.full(E, orc.global_scale_of(x), np.float32)
    c = dict(cfg=cfg, E=E, N=N, K=K, T=T, k=k, Wd=Wd, Wo=Wo, x=x, ids=ids, wts=wts, R=R, ga=ga)
    _cache[key] = c
    return c


def sample_rows(offsets, n_target, seed=0):
    """Permuted rows spanning every nonempty expert's first and last row (ragged tails) plus random
    rows, at most about n_target."""
    offsets = np.asarray(offsets)
    rows = set()
    for e in range(offsets.size - 1):
        if offsets[e + 1] > offsets[e]:
            rows.add(int(offsets[e]))
            rows.add(int(offsets[e + 1] - 1))
        if len(rows) >= n_target // 2:
            break
    rng = np.random.default_rng(seed)
    total = int(offsets[-1])
    extra = rng.choice(total, size=min(total, max(0, n_target - len(rows))), replace=False)
    rows.update(int(r) for r in extra)
    return np.array(sorted(rows), np.int64)


def sample_expert_rows(offsets, n_experts=3, per_expert=48, seed=0):
    """Rows of a few experts (the busiest, the least busy nonempty one, random others); per expert its
    first rows, its last row (a ragged tile tail) and random rows, at most per_expert each."""
    offsets = np.asarray(offsets)
    counts = np.diff(offsets)
    nz = np.flatnonzero(counts > 0)
    rng = np.random.default_rng(seed)
    pick = [int(nz[np.argmax(counts[nz])]), int(nz[np.argmin(counts[nz])])]
    others = [int(e) for e in rng.permutation(nz) if int(e) not in pick]
    pick += others[:max(0, n_experts - 2)]
    rows = set()
    for e in pick:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        cand = list(range(lo, min(hi, lo + 4))) + [hi - 1]
        extra = rng.choice(hi - lo, size=min(hi - lo, per_expert), replace=False) + lo
        for r in cand + [int(v) for v in extra]:
            if len([x for x in rows if lo <= x < hi]) >= per_expert:
                break
            rows.add(int(r))
    return np.array(sorted(rows), np.int64), sorted(pick)


def sample_tile_rows(offsets, n_experts=16, per_expert=64, seed=0, tile=128):
    """Rows of n_experts experts: the busiest one in full tile coverage (the first and last row of every
    `tile`-token tile, its last row, plus random rows), the least busy nonempty one and random others
    (their first rows, last row and random rows, at most per_expert each). Returns (rows, experts)."""
    offsets = np.asarray(offsets)
    counts = np.diff(offsets)
    nz = np.flatnonzero(counts > 0)
    rng = np.random.default_rng(seed)
    busiest = int(nz[np.argmax(counts[nz])])
    pick = [busiest, int(nz[np.argmin(counts[nz])])]
    pick += [int(e) for e in rng.permutation(nz) if int(e) not in pick][:max(0, n_experts - 2)]
    rows = set()
    lo, hi = int(offsets[busiest]), int(offsets[busiest + 1])
    for t0 in range(lo, hi, tile):
        rows.update((t0, min(hi, t0 + tile) - 1))
    rows.update(int(r) for r in rng.choice(np.arange(lo, hi), size=min(hi - lo, per_expert), replace=False))
    for e in pick[1:]:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        mine = set(range(lo, min(hi, lo + 4))) | {hi - 1}
        extra = rng.choice(np.arange(lo, hi), size=min(hi - lo, per_expert), replace=False)
        for r in extra:
            if len(mine) >= per_expert:
                break
            mine.add(int(r))
        rows |= mine
    return np.array(sorted(rows), np.int64), sorted(pick)


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def gamma_h_table(name):
    """The per-expert tensor scale of the MLP intermediate for a workload, written by the oracle-only
    script golden/make_gamma_h.py: (gamma_h [E] float32, amax_h [E] float32, routed rows [E])."""
    ent = {}
    with open(os.path.join(GOLDEN, "gamma_h.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            w = line.split()
            if w[0] == name:
                ent[int(w[1])] = (float.fromhex(w[3]), float.fromhex(w[2]), int(w[4]))
    E = len(ent)
    assert sorted(ent) == list(range(E)), "gamma_h table of %s is incomplete" % name
    g = np.array([ent[e][0] for e in range(E)], np.float32)
    a = np.array([ent[e][1] for e in range(E)], np.float32)
    n = np.array([ent[e][2] for e in range(E)], np.int64)
    return g, a, n
