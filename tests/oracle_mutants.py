"""Mutation check of the oracle's pins (test infrastructure; not collected by pytest).

Each entry below plants one plausible slip in a copy of ``oracle/`` (a
dropped term, a wrong sign, index, axis or rounding mode, a transposed
operand, a wrong default) and runs the CPU pin tests on that copy. Every
mutant must make at least one pin fail; the ones listed under EQUIVALENT
cannot, because they do not change what is computed, and are run only to
show that they survive for that reason.

Usage (from the repository root, CPU only, about a minute with 4 workers):

    python tests/oracle_mutants.py            # all mutants
    python tests/oracle_mutants.py 3 17 42    # some of them, by index

Exit status 1 if a non-equivalent mutant survives.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["test_oracle_pins.py", "test_oracle_yaqa.py", "test_oracle_deploy.py", "test_oracle_a4.py"]
K, Y, D = "kronq.py", "yaqa.py", "deploy.py"

# (file under oracle/, text to replace (must occur once), replacement)
MUTANTS = [
    (K, '<< np.uint32(16)).view',
     '<< np.uint32(15)).view'),
    (K, 'r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16',
     'r = (u + 0x8000) >> 16'),
    (K, 'r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16',
     'r = u >> 16'),
    (K, 'HX = xq.T @ xq / n',
     'HX = xq.T @ xq / (n - 1)'),
    (K, 'd32 = (x32 - xq32).astype(np.float32)',
     'd32 = (xq32 - x32).astype(np.float32)'),
    (K, 'D = d32.astype(np.float64).T @ xq / n',
     'D = xq.T @ d32.astype(np.float64) / n'),
    (K, '                d32 = bf16_rne(d32)',
     '                pass'),
    (K, 'HX = xq.T @ xq / n',
     'HX = (decode_inputs(X).astype(np.float64).T @ decode_inputs(X).astype(np.float64) / n) if X is not None else xq.T @ xq / n'),
    (K, 'ng = g.shape[0] if n_total is None else n_total',
     'ng = g.shape[0]'),
    (K, 'h = np.block([[h, h], [h, -h]])',
     'h = np.block([[h, h], [-h, h]])'),
    (K, 'return d & (-d)',
     'return min(d & (-d), 64)'),
    (K, 'hb = sylvester(b) / np.sqrt(b)',
     'hb = sylvester(b) / b'),
    (K, 'return apply_hadamard_left(M.T, sign, b).T',
     'return apply_hadamard_left(M.T, sign, b)'),
    (K, 'out[ok] = (diag_h[ok] / sq_norm[ok]) ** 0.25',
     'out[ok] = (diag_h[ok] / sq_norm[ok]) ** 0.5'),
    (K, 'out[ok] = (diag_h[ok] / sq_norm[ok]) ** 0.25',
     'out[ok] = (sq_norm[ok] / diag_h[ok]) ** 0.25'),
    (K, 'ok = (diag_h > 0) & (sq_norm > 0)',
     'ok = (diag_h > 0)'),
    (K, 'c = np.sum(W * W, axis=0)\n    r = np.sum(W * W, axis=1)',
     'c = np.sum(W * W, axis=1)\n    r = np.sum(W * W, axis=0)'),
    (K, 'W1 = s_g[:, None] * W * s_x[None, :]',
     'W1 = W / s_g[:, None] / s_x[None, :]'),
    (K, 'HX1 = np.asarray(HX, np.float64) / np.outer(s_x, s_x)',
     'HX1 = np.asarray(HX, np.float64) * np.outer(s_x, s_x)'),
    (K, 'HG1 = np.asarray(HG, np.float64) / np.outer(s_g, s_g)',
     'HG1 = np.asarray(HG, np.float64) * np.outer(s_g, s_g)'),
    (K, 'D1 = np.asarray(D, np.float64) / np.outer(s_x, s_x)',
     'D1 = np.asarray(D, np.float64)'),
    (K, 'W2 = apply_hadamard_right(apply_hadamard_left(W1, sign_out, bo), sign_in, bi)',
     'W2 = apply_hadamard_right(apply_hadamard_left(W1, sign_in, bo), sign_out, bi)'),
    (K, 'HG2 = apply_hadamard_right(apply_hadamard_left(HG1, sign_out, bo), sign_out, bo)',
     'HG2 = apply_hadamard_right(apply_hadamard_left(HG1, sign_in, bo), sign_in, bo)'),
    (K, 'D2 = apply_hadamard_right(apply_hadamard_left(D1, sign_in, bi), sign_in, bi)',
     'D2 = apply_hadamard_right(apply_hadamard_left(D1.T, sign_in, bi), sign_in, bi)'),
    (K, 'return tx, tg, tx * tg\n\n\ndef covariance_diagonals',
     'return tx, tg, tx + tg\n\n\ndef covariance_diagonals'),
    (K, 'dx = np.einsum("tj,tj->j", xq, xq) / n',
     'dx = np.einsum("tj,tj->j", xq, xq) / xq.shape[0]'),
    (K, 'tx = float(np.sum(dhx / (s_x * s_x)))',
     'tx = float(np.sum(dhx * (s_x * s_x)))'),
    (K, 'return H + damp * np.mean(np.diag(H)) * np.eye(H.shape[0])',
     'return H + damp * np.mean(H) * np.eye(H.shape[0])'),
    (K, 'return H + damp * np.mean(np.diag(H)) * np.eye(H.shape[0])',
     'return H + damp * np.eye(H.shape[0])'),
    (K, 'return np.linalg.cholesky(Hinv).T',
     'return np.linalg.cholesky(Hinv)'),
    (K, 'return np.linalg.cholesky(Hinv).T',
     'return np.linalg.inv(np.linalg.cholesky(Hd))'),
    (K, 'T = np.triu(np.asarray(D, np.float64) @ np.asarray(U, np.float64).T, 1)',
     'T = np.triu(np.asarray(D, np.float64) @ np.asarray(U, np.float64).T, 0)'),
    (K, 'T = np.triu(np.asarray(D, np.float64) @ np.asarray(U, np.float64).T, 1)',
     'T = np.triu(np.asarray(D, np.float64).T @ np.asarray(U, np.float64).T, 1)'),
    (K, 'return T @ np.asarray(U, np.float64)',
     'return T @ np.asarray(U, np.float64).T'),
    (K, 'T[r, k <= p] = 0.0',
     'T[r, k < p] = 0.0'),
    (K, 'lo = np.minimum(v.min(axis=1), np.float32(0))',
     'lo = v.min(axis=1)'),
    (K, 'hi = np.maximum(v.max(axis=1), np.float32(0))',
     'hi = v.max(axis=1)'),
    (K, 'zero = np.rint((-lo).astype(np.float32) / scale).astype(np.float32)',
     'zero = np.floor((-lo).astype(np.float32) / scale + np.float32(0.5)).astype(np.float32)'),
    (K, 'scale = ((hi - lo).astype(np.float32) / maxq).astype(np.float32)',
     'scale = ((hi - lo).astype(np.float32) / (maxq + 1)).astype(np.float32)'),
    (K, 'lo = np.where(same, np.float32(-1), lo).astype(np.float32)',
     'lo = np.where(same, np.float32(0), lo).astype(np.float32)'),
    (K, 'q = np.clip(np.rint(v) + zero.astype(np.float64), 0, maxq)',
     'q = np.clip(np.rint(v) + zero.astype(np.float64), 0, maxq - 1)'),
    (K, 'q = np.clip(np.rint(v) + zero.astype(np.float64), 0, maxq)',
     'q = np.clip(np.floor(v + 0.5) + zero.astype(np.float64), 0, maxq)'),
    (K, 'e = (w - wq) / U[p, p]',
     'e = (w - wq) * U[p, p]'),
    (K, 'e = (w - wq) / U[p, p]',
     'e = (wq - w) / U[p, p]'),
    (K, 'W[:, p + 1:b1] += np.outer(W0[:, p], P[p, p + 1:b1])',
     'W[:, p + 1:b1] += np.outer(W[:, p], P[p, p + 1:b1])'),
    (K, 'W[:, b1:] += W0[:, b0:b1] @ P[b0:b1, b1:]',
     'W[:, b1:] += W[:, b0:b1] @ P[b0:b1, b1:]'),
    (K, 'W[:, b1:] += W0[:, b0:b1] @ P[b0:b1, b1:]',
     'W[:, b1:] -= W0[:, b0:b1] @ P[b0:b1, b1:]'),
    (K, 'W[:, p + 1:b1] += np.outer(W0[:, p], P[p, p + 1:b1])',
     'W[:, p + 1:b1] -= np.outer(W0[:, p], P[p, p + 1:b1])'),
    (K, 'sc, zr = grid_fp32(W[:, p:min(p + group, n)].astype(np.float32), bits)',
     'sc, zr = grid_fp32(W0[:, p:min(p + group, n)].astype(np.float32), bits)'),
    (K, 'W[:, b1:] -= E @ U[b0:b1, b1:]',
     'W[:, b1:] -= E @ U[b0:b1, b1:] * 0.5'),
    (K, 'W[:, p + 1:b1] -= np.outer(e, U[p, p + 1:b1])',
     'W[:, p + 1:] -= np.outer(e, U[p, p + 1:])'),
    (K, 'sc, zr = grid_fp32(W0.astype(np.float32), bits)\n        scales',
     'sc, zr = grid_fp32(W0.astype(np.float32), bits + 1)\n        scales'),
    (K, 'mid = 0.5 * (q[i] + fq[i]) - zr[i]',
     'mid = 0.5 * (q[i] + fq[i])'),
    (K, 'M = M + 2.0 * (W0 @ np.asarray(D, np.float64))',
     'M = M + 1.0 * (W0 @ np.asarray(D, np.float64))'),
    (K, 'M = M + 2.0 * (W0 @ np.asarray(D, np.float64))',
     'M = M - 2.0 * (W0 @ np.asarray(D, np.float64))'),
    (K, 'M = M + 2.0 * (W0 @ np.asarray(D, np.float64))',
     'M = M + 2.0 * (W0 @ np.asarray(D, np.float64).T)'),
    (K, 'return float(np.max(np.abs(Q)))',
     'return float(np.max(np.abs(Q)) * np.sqrt(Q.shape[0]))'),
    (K, 'cn = np.sqrt(np.sum(W * W, axis=0))\n    rn = np.sqrt(np.sum(W * W, axis=1))',
     'cn = np.sqrt(np.sum(W * W, axis=1))\n    rn = np.sqrt(np.sum(W * W, axis=0))'),
    (K, 'return float(np.std(cn) / np.mean(cn)), float(np.std(rn) / np.mean(rn))',
     'return float(np.std(cn, ddof=1) / np.mean(cn)), float(np.std(rn, ddof=1) / np.mean(rn))'),
    (K, 'order = sorted(range(len(s)), key=lambda i: (-s[i], i))',
     'order = sorted(range(len(s)), key=lambda i: (s[i], i))'),
    (K, 'order = sorted(range(len(s)), key=lambda i: (-s[i], i))',
     'order = sorted(range(len(s)), key=lambda i: (-s[i], -i))'),
    (K, 'if used + extra <= budget:',
     'if used + extra < budget:'),
    (K, 'for w in reversed(ws):',
     'for w in ws:'),
    (K, 'HX, D, HG = [p if acc is None else (acc if p is None else acc + p)',
     'HX, D, HG = [p if acc is None else (acc if p is None else p)'),
    (K, 'res = sweep(W2, U, P, bits, group, block)',
     'res = sweep(W2, U, None, bits, group, block)'),
    (K, 'U = inv_factor(HX2, damp)',
     'U = inv_factor(HX, damp)'),
    (K, 'out[k, blk:blk + b] = (1 - 2 * par) * sign[blk:blk + b] / np.sqrt(b)',
     'out[k, blk:blk + b] = (1 - 2 * par) * sign[int(i)] / np.sqrt(b)'),
    (K, 'tx, tg, s = sensitivity(HX2, HG2)',
     'tx, tg, s = sensitivity(HX, HG)'),
    (Y, 'return R / r[None, :], r * r',
     'return R / r[:, None], r * r'),
    (Y, 'return R / r[None, :], r * r',
     'return R / r[None, :], r'),
    (Y, 'L = np.linalg.cholesky(H[::-1, ::-1])\n    R = L[::-1, ::-1]',
     'L = np.linalg.cholesky(H)\n    R = L.T'),
    (Y, 'q, W = rnd(Wt + Lo.T @ Dl @ Li + Lo.T @ Dl + Dl @ Li)\n    Dl',
     'q, W = rnd(Wt + Lo.T @ Dl + Dl @ Li)\n    Dl'),
    (Y, 'q, W = rnd(Wt + Lo.T @ Dl @ Li + Lo.T @ Dl + Dl @ Li)\n    Dl',
     'q, W = rnd(Wt + Lo @ Dl @ Li + Lo @ Dl + Dl @ Li)\n    Dl'),
    (Y, 'for _ in range(m + n - 1 if iters is None else iters):',
     'for _ in range(max(m, n) - 1 if iters is None else iters):'),
    (Y, 'base = Wt[i] - U_out[:i, i] @ M[:i]',
     'base = Wt[i] - U_out[i, :i] @ M[:i]'),
    (Y, 'base = Wt[i] - U_out[:i, i] @ M[:i]',
     'base = Wt[i] + U_out[:i, i] @ M[:i]'),
    (Y, 'z = base[j] - uo * t[j]',
     'z = base[j] - t[j]'),
    (Y, 'e[j] = (z - wq) / (uo * U_in[j, j])',
     'e[j] = (z - wq) / U_in[j, j]'),
    (Y, 't[j + 1:] += e[j] * U_in[j, j + 1:]',
     't[j + 1:] += e[j] * U_in[j + 1:, j]'),
    (Y, 'M[i] = e @ U_in',
     'M[i] = e @ U_in.T'),
    (Y, 'Wt = W0 if P is None else W0 + W0 @ np.asarray(P, dtype=np.float64)',
     'Wt = W0 if P is None else W0 - W0 @ np.asarray(P, dtype=np.float64)'),
    (Y, 'sc, zr = grid_fp32(W0.astype(np.float32), bits)',
     'sc, zr = grid_fp32(Wt.astype(np.float32), bits)'),
    (Y, 'return e * np.diag(U_out)[:, None] * np.diag(U_in)[None, :]',
     'return e * np.diag(U_in)[None, :]'),
    (Y, 'over = np.where(q == 0, r - 0.5, np.where(q == top, -r - 0.5, np.abs(r) - 0.5))',
     'over = np.abs(r) - 0.5'),
    (Y, 'mid = 0.5 * (q + fq) - z64',
     'mid = 0.5 * (q + fq)'),
    (D, 'return (w + 3) // 4 * 4',
     'return w'),
    (D, '        if sh + bits > 32:\n            out[:, w + 1] |= v >> np.uint64(32)',
     '        pass'),
    (D, 'v |= p[:, w + 1] << np.uint64(32 - sh)',
     'v |= p[:, w + 1] << np.uint64(sh)'),
    (D, 'return np.repeat(sc, gs, axis=1)[:, :q.shape[1]] * (q - np.repeat(zr, gs, axis=1)[:, :q.shape[1]])',
     'return np.tile(sc, (1, gs))[:, :q.shape[1]] * (q - np.tile(zr, (1, gs))[:, :q.shape[1]])'),
    (D, 'A = so[:, None] * apply_hadamard_left(Wp, np.ones(d_out), bo)',
     'A = apply_hadamard_left(Wp, so, bo)'),
    (D, 'return B / np.asarray(s_g, np.float64)[:, None] / np.asarray(s_x, np.float64)[None, :]',
     'return B * np.asarray(s_g, np.float64)[:, None] / np.asarray(s_x, np.float64)[None, :]'),
    (D, 'x1 = x / np.asarray(s_x, np.float64)[None, :]\n    x2 = apply_hadamard_left(x1.T, sign_in, bi)',
     'x1 = x * np.asarray(s_x, np.float64)[None, :]\n    x2 = apply_hadamard_left(x1.T, sign_in, bi)'),
    (D, 'y2 = np.asarray(sign_out, np.float64)[:, None] * apply_hadamard_left(y1, np.ones(d_out), bo)\n    return (y2',
     'y2 = apply_hadamard_left(y1, sign_out, bo)\n    return (y2'),
    (D, 'qmax = (1 << (bits - 1)) - 1',
     'qmax = (1 << bits) - 1'),
    (D, 'q = np.clip(np.rint(t), -qmax - 1, qmax).astype(np.int8)',
     'q = np.clip(np.rint(t), -qmax, qmax).astype(np.int8)'),
    (D, 'q = np.clip(np.rint(t), -qmax - 1, qmax).astype(np.int8)',
     'q = np.clip(np.floor(t + 0.5), -qmax - 1, qmax).astype(np.int8)'),
    (D, 'mx = np.max(np.abs(x), axis=1)',
     'mx = np.max(x, axis=1)'),
    (D, 'x1 = x / np.asarray(s_x, np.float64)[None, :]\n    return',
     'x1 = x * np.asarray(s_x, np.float64)[None, :]\n    return'),
    (D, 'xa = qa["s"].astype(np.float64)[:, None] * qa["q"].astype(np.float64)',
     'xa = qa["q"].astype(np.float64)'),
    (D, 's = (np.float32(clip) * mx).astype(np.float32) / np.float32(qmax)',
     's = (mx).astype(np.float32) / np.float32(qmax)'),
    (K, 'dW = W0 - np.asarray(What, np.float64)',
     'dW = np.asarray(What, np.float64) - W0'),
    (K, 'bi = blk_in or hadamard_block(d_in)\n    bo = blk_out or hadamard_block(d_out)\n    c =',
     'bi = blk_in or hadamard_block(d_out)\n    bo = blk_out or hadamard_block(d_in)\n    c ='),
    (K, 'tx, tg, s = sensitivity(HX2, HG2)',
     'tx, tg, s = sensitivity(damped(HX2, damp), HG2)'),
    (K, 'codes_rtn, what_rtn = rtn(W2, bits, group)',
     'codes_rtn, what_rtn = rtn(W, bits, group)'),
    (K, 'g = p // group if group else 0',
     'g = (p // group) % 2 if group else 0'),
    (K, 'par ^= bits & 1',
     'par |= bits & 1'),
    (K, 'n_groups = (n + group - 1) // group if group else 1',
     'n_groups = n // group if group else 1'),
    (K, 'wq = sc.astype(np.float64) * (q - zr.astype(np.float64))\n            codes',
     'wq = sc.astype(np.float64) * q\n            codes'),
    (K, 'what[:, g0:g1] = sc[:, None].astype(np.float64) * (q - zr[:, None].astype(np.float64))',
     'what[:, g0:g1] = sc[:, None].astype(np.float64) * q'),
    (K, 'sc, zr = grid_fp32(W0[:, g0:g1].astype(np.float32), bits)',
     'sc, zr = grid_fp32(W0.astype(np.float32), bits)'),
    (D, 'bit = bits * j\n        w, sh = bit // 32, bit % 32\n        v = codes',
     'bit = bits * j + (j // 32)\n        w, sh = bit // 32, bit % 32\n        v = codes'),
    (D, 't[nz] = x[nz] / s[nz, None]',
     't[nz] = x[nz] * (np.float32(1) / s[nz, None])'),
]

# mutants that change nothing that is computed, with the reason
EQUIVALENT = [
    (K, 'return float(np.sum(np.asarray(HG, np.float64) * K.T))',
     'return float(np.sum(np.asarray(HG, np.float64) * K))',
     'H_G is symmetric, so sum(H_G * K) equals sum(H_G * K^T)'),
    (K, 'Hinv = 0.5 * (Hinv + Hinv.T)',
     'Hinv = np.triu(Hinv) + np.triu(Hinv, 1).T',
     "both symmetrizations of the fp64 inverse agree to rounding, far below any pin's tolerance"),
    (Y, 'return float(np.sum((dW @ np.asarray(H_in, np.float64) @ dW.T) * np.asarray(H_out, np.float64)))',
     'return float(np.sum((dW @ np.asarray(H_in, np.float64) @ dW.T) * np.asarray(H_out, np.float64).T))',
     'H_out is symmetric, so the transpose changes nothing'),
]


def run_one(f, old, new):
    """Copy the oracle, the seeded generators and the pins, plant the slip,
    run the pins. Returns (status, first failing test or the summary)."""
    d = tempfile.mkdtemp(prefix="oracle_mutant_")
    try:
        skip = shutil.ignore_patterns("__pycache__")
        shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(d, "oracle"), ignore=skip)
        shutil.copytree(os.path.join(ROOT, "synth"), os.path.join(d, "synth"), ignore=skip)
        shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(d, "tests", "golden"))
        for t in PINS + ["conftest.py"]:
            shutil.copy(os.path.join(ROOT, "tests", t), os.path.join(d, "tests", t))
        path = os.path.join(d, "oracle", f)
        with open(path) as fh:
            src = fh.read()
        if src.count(old) != 1:
            return "BAD PATTERN", f"found {src.count(old)} times"
        with open(path, "w") as fh:
            fh.write(src.replace(old, new))
        env = dict(os.environ, OMP_NUM_THREADS="2", OPENBLAS_NUM_THREADS="2",
                   PYTHONDONTWRITEBYTECODE="1")
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            "-m", "not gpu"] + [os.path.join("tests", t) for t in PINS],
                           cwd=d, env=env, capture_output=True, text=True, timeout=600)
        out = [ln for ln in r.stdout.splitlines() if ln.strip()]
        failed = [ln for ln in out if ln.startswith(("FAILED", "ERROR"))]
        return ("KILLED" if r.returncode else "SURVIVED"), (failed or out[-1:] or [""])[0]
    finally:
        shutil.rmtree(d, ignore_errors=True)


def main():
    cases = [(i, m[:3], False) for i, m in enumerate(MUTANTS)]
    cases += [(len(MUTANTS) + i, m[:3], True) for i, m in enumerate(EQUIVALENT)]
    sel = {int(a) for a in sys.argv[1:]}
    cases = [c for c in cases if not sel or c[0] in sel]
    with cf.ProcessPoolExecutor(4) as ex:
        futs = {c[0]: ex.submit(run_one, *c[1]) for c in cases}
        bad = []
        for i, (f, old, new), equivalent in cases:
            st, info = futs[i].result()
            tag = "equivalent " if equivalent else ""
            print(f"{i:3d} {tag}{st:9s} {f}: {old.strip()[:50]!r} -> {new.strip()[:40]!r} | {info[:90]}",
                  flush=True)
            if st != "KILLED" and not equivalent:
                bad.append(i)
    print(f"{len(cases)} mutants run; surviving non-equivalent: {bad}")
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main())
