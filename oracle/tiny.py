"""Independent brute-force oracle for tiny inputs.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``).  Pure Python: plain
loops over lists, every sum through ``math.fsum`` (the exactly rounded sum of
its terms), no numpy arithmetic and nothing shared with ``oracle.c``.  It
exists to pin the C oracle to a second implementation written from the same
definitions: the tests compare the two at 1e-12 on random shapes with every
size at most 32.

Definitions (the pages' formulas, in the notation of the tests):
  * RMSNorm (devpress.csdn.net explainer of "Defeating Nondeterminism in LLM
    Inference", section 3.1; eps from tom-jerr.github.io "Batch-Invariant
    Kernel", section RMSNorm): y[i][j] = x[i][j] / sqrt(mean_j x[i][j]^2 + eps)
    * gamma[j].
  * GEMM (the same explainer, section 3.2): C[i][j] = sum_k A[i][k] W[k][j].
  * Attention (section 3.3; "Batch-Invariant Kernel", section Flash
    Attention): row i at position pos[i] of query head h sees keys 0..pos[i]
    of KV head h // (Hq / Hkv); softmax of scale * q.k, weighted sum of v.
  * Chunked attention: keys split into chunks of a fixed size counted from
    position 0; per chunk the partial (m, l, o) with m the chunk's max score,
    l the sum of exp(s - m), o the exp-weighted sum of v; partials merged by a
    binary tree over 2**depth leaves, leaves past the last chunk the identity
    (-inf, 0, 0), each merge m = max(m1, m2), a_i = exp(m_i - m),
    l = a1 l1 + a2 l2, o = a1 o1 + a2 o2; output o / l.
"""
import math

NEG_INF = float("-inf")


def rmsnorm(x, gamma, eps):
    """x: list of rows (lists of floats), gamma: list; returns list of rows."""
    out = []
    for row in x:
        d = len(row)
        r = math.sqrt(math.fsum(v * v for v in row) / d + eps)
        out.append([row[j] / r * gamma[j] for j in range(d)])
    return out


def gemm(a, w):
    """a: M rows of K, w: K rows of N; returns M rows of N."""
    K = len(w)
    N = len(w[0]) if K else 0
    return [[math.fsum(a[i][k] * w[k][j] for k in range(K)) for j in range(N)]
            for i in range(len(a))]


def _scores(qv, keys, scale):
    return [scale * math.fsum(qv[e] * kv[e] for e in range(len(qv))) for kv in keys]


def attention(q, pos, k, v, scale):
    """q[i][h] (lists of D), pos[i], k[t][g], v[t][g]; returns out[i][h]."""
    Hq = len(q[0])
    Hkv = len(k[0])
    G = Hq // Hkv
    out = []
    for i, p in enumerate(pos):
        rows = []
        for h in range(Hq):
            g = h // G
            keys = [k[t][g] for t in range(p + 1)]
            vals = [v[t][g] for t in range(p + 1)]
            s = _scores(q[i][h], keys, scale)
            m = max(s)
            wts = [math.exp(x - m) for x in s]
            den = math.fsum(wts)
            D = len(vals[0])
            rows.append([math.fsum(wts[t] * vals[t][e] for t in range(len(vals))) / den
                         for e in range(D)])
        out.append(rows)
    return out


def _combine(a, b):
    ma, la, oa = a
    mb, lb, ob = b
    m = max(ma, mb)
    if m == NEG_INF:
        return (NEG_INF, 0.0, [0.0] * len(oa))
    fa = 0.0 if ma == NEG_INF else math.exp(ma - m)
    fb = 0.0 if mb == NEG_INF else math.exp(mb - m)
    return (m, fa * la + fb * lb, [fa * oa[e] + fb * ob[e] for e in range(len(oa))])


def attention_chunked(q, pos, k, v, scale, chunk, depth):
    """The chunked form above; returns out[i][h]."""
    Hq = len(q[0])
    Hkv = len(k[0])
    G = Hq // Hkv
    D = len(q[0][0])
    out = []
    for i, p in enumerate(pos):
        rows = []
        for h in range(Hq):
            g = h // G
            leaves = []
            n_chunks = p // chunk + 1
            assert n_chunks <= 2 ** depth
            for c in range(2 ** depth):
                lo, hi = c * chunk, min((c + 1) * chunk, p + 1)
                if c >= n_chunks or lo >= hi:
                    leaves.append((NEG_INF, 0.0, [0.0] * D))
                    continue
                s = _scores(q[i][h], [k[t][g] for t in range(lo, hi)], scale)
                m = max(s)
                wts = [math.exp(x - m) for x in s]
                o = [math.fsum(wts[t] * v[lo + t][g][e] for t in range(hi - lo))
                     for e in range(D)]
                leaves.append((m, math.fsum(wts), o))
            level = leaves
            while len(level) > 1:
                level = [_combine(level[2 * j], level[2 * j + 1]) for j in range(len(level) // 2)]
            m, l, o = level[0]
            rows.append([x / l for x in o])
        out.append(rows)
    return out


def chunk_partition(n_keys, chunk):
    """Valid keys in each chunk of keys 0..n_keys-1 (chunks from position 0)."""
    counts = []
    start = 0
    while start < n_keys:
        counts.append(min(chunk, n_keys - start))
        start += chunk
    return counts


def round_bf16(x):
    """The bf16 value nearest to x (ties to an even significand), straight from x."""
    if x != x or x in (float("inf"), float("-inf")) or x == 0.0:
        return x
    mant, exp = math.frexp(abs(x))            # abs(x) = mant * 2**exp, mant in [0.5, 1)
    # 8 significant bits (1 + 7 stored) above the normal range's floor; the
    # subnormal spacing 2**-133 below it
    quantum_exp = max(exp - 8, -133)
    q = math.ldexp(1.0, quantum_exp)
    r = round(abs(x) / q) * q                 # abs(x) / q is exact; round() ties to even
    if r >= math.ldexp(1.0, 128):             # rounded past the largest bf16, 255 * 2**120
        r = float("inf")
    return math.copysign(r, x)
