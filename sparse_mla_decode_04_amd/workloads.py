"""Seeded synthetic inputs for sparse NVFP4 MLA decode.

This module only draws random numbers and index lists; it holds none of the
method's arithmetic (no quantization, no attention).  It is the one piece of
Python shared by the GPU path's tests/benchmark and the CPU oracle's tests:
both sides receive exactly the same fp16 source rows, queries and index lists.

The five named workloads reproduce the shapes of the serving scenario on the
pages ("Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily":
a 35-token sparse-attention launch over 2,048-entry index lists in "Four-bit
caches make room"; ~140K-token agent prompts plus ~6K new tokens in "Why
agents strain inference servers"; 66 concurrent sessions in "Split the prompt
from generation"; 1.63M cached tokens per decoder in "Four-bit caches make
room").  They stand in for the AgentX agent-session replay the vendor blog
benchmarks with; none of that benchmark's data is used.

Every pool row's fp16 source values are N(0,1) and depend only on
(workload seed, row id): rows are generated in fixed chunks of CHUNK_ROWS
rows, each chunk from its own seeded stream, so any subset of rows can be
regenerated without generating the whole pool.
"""

from dataclasses import dataclass, field

import numpy as np

HEAD_DIM = 576          # 512 latent + 64 rope values per cache row / query head
TOPK = 2048             # entries per index list
CHUNK_ROWS = 8192       # pool rows per independently seeded chunk

# stream ids under a workload seed
_S_POOL, _S_Q, _S_OFFSETS, _S_INDICES, _S_EMPTIES, _S_NEWROWS, _S_SLOTS, _S_SCORES = range(8)


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    T: int                    # decode tokens
    H: int                    # query heads
    pool_rows: int            # cache rows in the pool
    topk: int = TOPK
    softmax_scale: float = 1.0 / 24.0   # 1/sqrt(576)
    kind: str = "uniform"     # index-list recipe
    params: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def seed(self):
        return 1000 + self.cfg_id


WORKLOADS = {
    1: Workload("tiny", 1, T=1, H=16, pool_rows=4096, kind="tiny",
                params={"empties_tail": 300}),
    2: Workload("small_batch_latency", 2, T=35, H=16, pool_rows=262144, kind="ranged",
                params={"context": 140000, "max_empty": 204}),
    3: Workload("medium_batch", 3, T=128, H=64, pool_rows=1048576, kind="clustered",
                params={"context": 146000, "recent": 8192, "recent_frac": 0.7,
                        "n_min": 256, "n_max": 2048}),
    4: Workload("agent_mix", 4, T=264, H=16, pool_rows=1630000, kind="sessions",
                params={"sessions": 66, "tokens_per_session": 4, "context": 146000,
                        "shared": 1536}),
    5: Workload("throughput_cache_write", 5, T=1024, H=128, pool_rows=1630000, kind="uniform",
                params={"new_rows": 1024}),
}


def custom(T, H, pool_rows, topk=TOPK, empty_frac=0.0, seed=7, name="custom"):
    """A small ad-hoc workload: per-token distinct uniform indices with a
    fraction of entries set to -1 at random positions."""
    return Workload(name, seed - 1000, T=T, H=H, pool_rows=pool_rows, topk=topk, kind="custom",
                    params={"empty_frac": float(empty_frac)})


def _rng(wl, stream, *extra):
    return np.random.default_rng([wl.seed, stream, *extra])


def pool_source(wl, rows=None):
    """fp16 [n, 576] N(0,1) source values of pool rows (all rows if `rows` is None)."""
    if rows is None:
        rows = np.arange(wl.pool_rows, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= wl.pool_rows):
        raise IndexError("row id out of range")
    out = np.empty((rows.size, HEAD_DIM), dtype=np.float16)
    if rows.size == 0:
        return out
    chunks = rows // CHUNK_ROWS
    for c in np.unique(chunks):
        sel = np.nonzero(chunks == c)[0]
        out[sel] = _chunk(wl, int(c))[rows[sel] - c * CHUNK_ROWS]
    return out


def _chunk(wl, c):
    n = min(CHUNK_ROWS, wl.pool_rows - c * CHUNK_ROWS)
    g = _rng(wl, _S_POOL, c)
    return g.standard_normal((n, HEAD_DIM), dtype=np.float32).astype(np.float16)


def pool_source_chunks(wl):
    """Yield (first_row, fp16 [n, 576]) chunks covering the whole pool, in order."""
    for c in range((wl.pool_rows + CHUNK_ROWS - 1) // CHUNK_ROWS):
        yield c * CHUNK_ROWS, _chunk(wl, c)


def queries(wl):
    """fp16 [T, H, 576] N(0,1) query vectors."""
    g = _rng(wl, _S_Q)
    return g.standard_normal((wl.T, wl.H, HEAD_DIM), dtype=np.float32).astype(np.float16)


def _distinct(g, lo, hi, k):
    """k distinct ints drawn uniformly from [lo, hi), in draw order."""
    return (lo + g.choice(hi - lo, size=k, replace=False)).astype(np.int64)


def index_lists(wl):
    """int32 [T, topk] index lists; -1 marks an empty entry."""
    T, K, N, p = wl.T, wl.topk, wl.pool_rows, wl.params
    idx = np.full((T, K), -1, dtype=np.int64)
    if wl.kind == "tiny":
        g = _rng(wl, _S_INDICES)
        idx[0] = _distinct(g, 0, N, K)
        idx[0, K - p["empties_tail"]:] = -1
    elif wl.kind == "ranged":
        go, gi, ge = _rng(wl, _S_OFFSETS), _rng(wl, _S_INDICES), _rng(wl, _S_EMPTIES)
        for t in range(T):
            off = int(go.integers(0, N - p["context"] + 1))
            idx[t] = _distinct(gi, off, off + p["context"], K)
            ne = int(ge.integers(0, p["max_empty"] + 1))
            idx[t, ge.choice(K, size=ne, replace=False)] = -1
    elif wl.kind == "clustered":
        go, gi = _rng(wl, _S_OFFSETS), _rng(wl, _S_INDICES)
        for t in range(T):
            off = int(go.integers(0, N - p["context"] + 1))
            n = int(gi.integers(p["n_min"], p["n_max"] + 1))
            n_recent = int(round(p["recent_frac"] * n))
            recent_lo = off + p["context"] - p["recent"]
            a = _distinct(gi, recent_lo, off + p["context"], n_recent)
            b = _distinct(gi, off, recent_lo, n - n_recent)
            v = np.concatenate([a, b])
            gi.shuffle(v)
            idx[t, :n] = v
    elif wl.kind == "sessions":
        go, gi = _rng(wl, _S_OFFSETS), _rng(wl, _S_INDICES)
        S, tps, sh = p["sessions"], p["tokens_per_session"], p["shared"]
        own = K - sh
        for s in range(S):
            off = int(go.integers(0, N - p["context"] + 1))
            pick = _distinct(gi, off, off + p["context"], sh + tps * own)
            shared = pick[:sh]
            for j in range(tps):
                v = np.concatenate([shared, pick[sh + j * own: sh + (j + 1) * own]])
                gi.shuffle(v)
                idx[s * tps + j] = v
    elif wl.kind == "uniform":
        gi = _rng(wl, _S_INDICES)
        for t in range(T):
            idx[t] = _distinct(gi, 0, N, K)
    elif wl.kind == "custom":
        gi, ge = _rng(wl, _S_INDICES), _rng(wl, _S_EMPTIES)
        k_draw = min(K, N)
        for t in range(T):
            idx[t, :k_draw] = _distinct(gi, 0, N, k_draw)
            ge.shuffle(idx[t])
            ne = int(round(p["empty_frac"] * K))
            if ne:
                idx[t, ge.choice(K, size=ne, replace=False)] = -1
    else:
        raise ValueError(wl.kind)
    return idx.astype(np.int32)


def indexer_inputs(wl):
    """Synthetic sparse-indexer inputs over each token's context: (scores float32 [T, S],
    lengths int32 [T], row_offset int32 [T]).  The context is the pool range the token's
    index list is drawn from (same offsets as index_lists; S = the context length).
    Scores are N(0,1) on a grid of 1/64, so many positions tie at the top-2,048 cut.
    Defined for the workloads whose tokens have a context range."""
    T, N, p = wl.T, wl.pool_rows, wl.params
    go = _rng(wl, _S_OFFSETS)
    if wl.kind == "ranged":
        offs = [int(go.integers(0, N - p["context"] + 1)) for _ in range(T)]
    elif wl.kind == "sessions":
        tps = p["tokens_per_session"]
        offs = np.repeat([int(go.integers(0, N - p["context"] + 1)) for _ in range(p["sessions"])], tps)
    else:
        raise ValueError(f"no context ranges in workload {wl.name}")
    S = p["context"]
    g = _rng(wl, _S_SCORES)
    scores = np.empty((T, S), dtype=np.float32)
    for t in range(T):
        scores[t] = np.round(g.standard_normal(S) * 64.0) / 64.0
    return scores, np.full(T, S, dtype=np.int32), np.asarray(offs, dtype=np.int32)


def new_rows(wl):
    """(fp16 [n, 576] N(0,1) rows, int32 [n] distinct slots) written into the pool
    before decode (the cache write of the throughput workload)."""
    n = wl.params.get("new_rows", 0)
    src = _rng(wl, _S_NEWROWS).standard_normal((n, HEAD_DIM), dtype=np.float32).astype(np.float16)
    slots = _distinct(_rng(wl, _S_SLOTS), 0, wl.pool_rows, n).astype(np.int32)
    return src, slots
