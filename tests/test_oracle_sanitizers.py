"""The C oracles under AddressSanitizer and UndefinedBehaviorSanitizer (CPU tier).

A small C driver is compiled with gcc together with the oracle sources, with both
sanitizers on, and run as a child process on a packed case (a long slot crossing the
64-token checkpoint boundary of the backward, an empty slot, a short slot, a tail of
unowned rows) and a dense GVA case, forward and backward, with two worker threads. The
sanitizers abort on the first report; the run must exit cleanly and its outputs must
equal those of the regular build bit for bit (same C, no fast-math, no FMA contraction).
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_DIR = os.path.join(os.path.dirname(HERE), "oracle")

DRIVER = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int kda_oracle_recurrent(const double*, const double*, const double*, const double*, const double*,
                         const double*, const int32_t*, int, double*, double*, int, int, int, int,
                         int, int, double, int);
int kda_oracle_recurrent_bwd(const double*, const double*, const double*, const double*,
                             const double*, const double*, const int32_t*, int, const double*,
                             const double*, double*, double*, double*, double*, double*, double*,
                             double*, double*, int, int, int, int, int, int, double, int);

static void* rd(const char* dir, const char* name, size_t n, size_t sz) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s.bin", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) { fprintf(stderr, "missing %s\n", path); exit(2); }
    void* p = malloc(n * sz ? n * sz : 1);
    if (n && fread(p, sz, n, f) != n) { fprintf(stderr, "short %s\n", path); exit(2); }
    fclose(f);
    return p;
}

static void wr(const char* dir, const char* name, const double* p, size_t n) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s.out", dir, name);
    FILE* f = fopen(path, "wb");
    fwrite(p, sizeof(double), n, f);
    fclose(f);
}

int main(int argc, char** argv) {
    if (argc != 10) return 2;
    const char* dir = argv[1];
    const int B = atoi(argv[2]), T = atoi(argv[3]), H = atoi(argv[4]), HV = atoi(argv[5]);
    const int K = atoi(argv[6]), V = atoi(argv[7]), N = atoi(argv[8]), packed = atoi(argv[9]);
    const size_t rows = (size_t)B * T;
    double* q = rd(dir, "q", rows * H * K, 8);
    double* k = rd(dir, "k", rows * H * K, 8);
    double* v = rd(dir, "v", rows * HV * V, 8);
    double* g = rd(dir, "g", rows * HV * K, 8);
    double* beta = rd(dir, "beta", rows * HV, 8);
    double* h0 = rd(dir, "h0", (size_t)N * HV * K * V, 8);
    double* dout = rd(dir, "dout", rows * HV * V, 8);
    double* dht = rd(dir, "dht", (size_t)N * HV * K * V, 8);
    int32_t* cu = packed ? rd(dir, "cu", (size_t)N + 1, 4) : NULL;
    double* sc = rd(dir, "scale", 1, 8);   /* the regular oracle's default, K ** -0.5 */
    const double scale = sc[0];
    free(sc);

    double* o = malloc(rows * HV * V * 8);
    for (size_t i = 0; i < rows * HV * V; ++i) o[i] = NAN;
    double* ht = calloc((size_t)N * HV * K * V, 8);
    int rc = kda_oracle_recurrent(q, k, v, g, beta, h0, cu, N, o, ht, B, T, H, HV, K, V, scale, 2);
    if (rc != 0) { fprintf(stderr, "forward rc %d\n", rc); return 3; }
    wr(dir, "o", o, rows * HV * V);
    wr(dir, "ht", ht, (size_t)N * HV * K * V);

    double* dq = calloc(rows * H * K, 8);
    double* dk = calloc(rows * H * K, 8);
    double* dv = calloc(rows * HV * V, 8);
    double* dg = calloc(rows * HV * K, 8);
    double* db = calloc(rows * HV, 8);
    double* dh0 = calloc((size_t)N * HV * K * V, 8);
    double* dq_hv = calloc(rows * HV * K, 8);
    double* dk_hv = calloc(rows * HV * K, 8);
    rc = kda_oracle_recurrent_bwd(q, k, v, g, beta, h0, cu, N, dout, dht, dq, dk, dv, dg, db, dh0,
                                  dq_hv, dk_hv, B, T, H, HV, K, V, scale, 2);
    if (rc != 0) { fprintf(stderr, "backward rc %d\n", rc); return 4; }
    wr(dir, "dq", dq, rows * H * K);
    wr(dir, "dk", dk, rows * H * K);
    wr(dir, "dv", dv, rows * HV * V);
    wr(dir, "dg", dg, rows * HV * K);
    wr(dir, "dbeta", db, rows * HV);
    wr(dir, "dh0", dh0, (size_t)N * HV * K * V);
    free(q); free(k); free(v); free(g); free(beta); free(h0); free(dout); free(dht); free(cu);
    free(o); free(ht); free(dq); free(dk); free(dv); free(dg); free(db); free(dh0);
    free(dq_hv); free(dk_hv);
    return 0;
}
"""

SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    d = tmp_path_factory.mktemp("oracle_san")
    src = d / "driver.c"
    src.write_text(DRIVER)
    exe = d / "driver"
    cmd = ["gcc", "-O1", "-g", "-std=c99", "-pthread", *SAN_FLAGS, str(src),
           os.path.join(ORACLE_DIR, "kda_oracle.c"), os.path.join(ORACLE_DIR, "kda_oracle_bwd.c"),
           "-lm", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitize" in r.stderr:
        pytest.skip("gcc here cannot link the sanitizer runtimes: " + r.stderr[-200:])
    assert r.returncode == 0, r.stderr
    return str(exe)


def _case(B, T, H, HV, K, V, cu, seed):
    rng = np.random.default_rng(seed)
    N = len(cu) - 1 if cu is not None else B
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    return dict(q=q, k=k, v=rng.standard_normal((B, T, HV, V)),
                g=np.log2(1.0 / (1.0 + np.exp(-rng.normal(2.0, 1.0, (B, T, HV, K))))),
                beta=1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, HV)))),
                h0=0.05 * rng.standard_normal((N, HV, K, V)),
                dout=rng.standard_normal((B, T, HV, V)), dht=rng.standard_normal((N, HV, K, V)),
                cu=None if cu is None else np.asarray(cu, dtype=np.int32), N=N)


@pytest.mark.parametrize("B,T,H,HV,K,V,cu", [
    (1, 160, 1, 2, 8, 4, [0, 70, 70, 75, 150]),   # long slot across the checkpoint, empty, short; tail
    (2, 67, 2, 4, 16, 8, None),                   # dense, GVA 2
])
def test_oracle_clean_under_sanitizers(driver, tmp_path, B, T, H, HV, K, V, cu):
    c = _case(B, T, H, HV, K, V, cu, seed=B * 100 + T)
    for name in ("q", "k", "v", "g", "beta", "h0", "dout", "dht"):
        np.ascontiguousarray(c[name], dtype=np.float64).tofile(tmp_path / f"{name}.bin")
    np.array([K ** -0.5], dtype=np.float64).tofile(tmp_path / "scale.bin")
    if cu is not None:
        c["cu"].tofile(tmp_path / "cu.bin")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([driver, str(tmp_path), str(B), str(T), str(H), str(HV), str(K), str(V),
                        str(c["N"]), str(int(cu is not None))], capture_output=True, text=True, env=env,
                       timeout=120)
    assert r.returncode == 0, f"sanitized oracle failed ({r.returncode}):\n{r.stderr[-3000:]}"

    def out(name, shape):
        return np.fromfile(tmp_path / f"{name}.out", dtype=np.float64).reshape(shape)

    N = c["N"]
    o_ref, ht_ref = oracle.recurrent(c["q"], c["k"], c["v"], c["g"], c["beta"], c["h0"], c["cu"])
    assert np.array_equal(out("o", o_ref.shape), o_ref, equal_nan=True)
    assert np.array_equal(out("ht", (N, HV, K, V)), ht_ref)
    ref = oracle.recurrent_bwd(c["q"], c["k"], c["v"], c["g"], c["beta"], c["dout"], c["h0"], c["cu"], c["dht"])
    for name, want in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), ref):
        assert np.array_equal(out(name, want.shape), want), name


def test_sanitizer_catches_a_planted_overrun(driver, tmp_path):
    """The same flags turn a one-past-the-end read into a failed run (the instrumentation
    is active, so a clean oracle run means something)."""
    src = tmp_path / "overrun.c"
    src.write_text("#include <stdlib.h>\nint main(void) { volatile double* p = malloc(8 * sizeof(double));\n"
                   "  for (int i = 0; i < 8; ++i) p[i] = i;\n  double s = p[8];\n  free((void*)p);\n"
                   "  return s > 1e300; }\n")
    exe = tmp_path / "overrun"
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", *SAN_FLAGS, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60,
                       env=dict(os.environ, ASAN_OPTIONS="halt_on_error=1"))
    # whichever sanitizer reports it first (UBSan's object-size check or ASan)
    assert r.returncode != 0 and ("heap-buffer-overflow" in r.stderr or "runtime error" in r.stderr)
