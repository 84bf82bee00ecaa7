"""How large the gradient errors of the attention backward would be if P and dS entered the gradient products as
one bf16 value instead of the hi + lo pair the kernels use (CPU, numpy, fp64 arithmetic apart from the rounding).

    python ceilings/bwd_rounding.py [seq]        # default 65536

Workload: one KV head with 4 query heads (the 32/8 GQA layer), head_dim 128, Q/K/V/dO iid N(0,1) rounded to
bf16, block-sparse causal keys (block 64, sink 128, window 2048).  For the sink key 0, a key near the start, one
in the middle and one near the end it sums dV = sum_i P_ij dO_i and dK = scale sum_i dS_ij Q_i over the query heads,
and for a few query rows dQ = scale sum_j dS_ij K_j, three ways: exact, with P / dS rounded to bf16
(round-to-nearest-even), and with the hi + lo pair (hi = truncation, lo = bf16(x - hi)).  Prints the max-abs error
of each against the exact sums; the parity bar of the gradients is max-abs 1e-2.
"""
import sys
import numpy as np


def bf16_rne(x):
    b = np.ascontiguousarray(x, np.float32).view(np.uint32)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.view(np.float32).astype(np.float64)


def bf16_trunc(x):
    return (np.ascontiguousarray(x, np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32).astype(np.float64)


def hi_lo(x):
    hi = bf16_trunc(x)
    return hi + bf16_rne(x - hi)


def fp16_rne(x):
    return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def main(S=65536, H=4, d=128, blk=64, sink=128, win=2048, seed=5):
    rng = np.random.default_rng(seed)
    k = bf16_rne(rng.standard_normal((S, d)))
    v = bf16_rne(rng.standard_normal((S, d)))
    scale = 1 / np.sqrt(d)
    probe_keys = [0, 100, S // 2, S - 70]
    probe_rows = [70, 5000, S // 2 + 3, S - 1]
    ways = {"exact": lambda x: x, "bf16": bf16_rne, "hi+lo": hi_lo, "fp16": fp16_rne}
    dv = {w: np.zeros((len(probe_keys), d)) for w in ways}
    dk = {w: np.zeros((len(probe_keys), d)) for w in ways}
    dq = {w: [] for w in ways}
    for h in range(H):
        q = bf16_rne(rng.standard_normal((S, d)))
        do = bf16_rne(rng.standard_normal((S, d)))
        for qb in range(S // blk):
            rows = np.arange(qb * blk, (qb + 1) * blk)
            kbs = sorted(set(range(min(sink // blk, qb + 1))) | set(range(max(0, qb - win // blk + 1), qb + 1)))
            keys = np.concatenate([np.arange(b * blk, (b + 1) * blk) for b in kbs])
            s = np.where(keys[None, :] <= rows[:, None], q[rows] @ k[keys].T * scale, -np.inf)
            p = np.exp(s - s.max(1, keepdims=True))
            p /= p.sum(1, keepdims=True)
            o = p @ v[keys]
            ds = p * (do[rows] @ v[keys].T - (do[rows] * o).sum(1, keepdims=True))
            for n, j in enumerate(probe_keys):
                c = np.nonzero(keys == j)[0]
                if len(c):
                    for w, f in ways.items():
                        dv[w][n] += f(p[:, c[0]]) @ do[rows]
                        dk[w][n] += scale * f(ds[:, c[0]]) @ q[rows]
            for r in probe_rows:
                if r in rows:
                    i = r - rows[0]
                    for w, f in ways.items():
                        dq[w].append(scale * f(ds[i]) @ k[keys])
    out = {}
    for name, g in (("dV", dv), ("dK", dk), ("dQ", {w: np.array(x) for w, x in dq.items()})):
        ex = g["exact"]
        out[name] = {"max_abs_value": float(np.abs(ex).max()),
                     "err_bf16": float(np.abs(g["bf16"] - ex).max()),
                     "err_hi_lo": float(np.abs(g["hi+lo"] - ex).max()),
                     "err_fp16": float(np.abs(g["fp16"] - ex).max())}
    return out


if __name__ == "__main__":
    S = int(sys.argv[1]) if len(sys.argv) > 1 else 65536
    for name, r in main(S).items():
        print(f"seq {S} {name}: max |exact| {r['max_abs_value']:.3f}   max-abs error, P/dS as one bf16: "
              f"{r['err_bf16']:.2e}   as hi + lo: {r['err_hi_lo']:.2e}   as one fp16: {r['err_fp16']:.2e}")
