"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host code only).

A small C driver calls o1_bwd_fwd and o1_fwd in every mode and branch on shapes
with tail chunks, GQA, odd ranks and chunk size 1, with arrays allocated to
their exact sizes; any out-of-bounds access, leak or undefined operation in
o1_contract.c aborts the run.
"""

import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent

DRIVER = r"""
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <math.h>

int o1_bwd_fwd(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
               int, int, int, int, const double *, const double *, const double *, const double *,
               const double *, const double *, const double *, const double *, const double *,
               const double *, const double *, const double *, const double *, const double *,
               const double *, const double *, const double *, double *, double *, double *,
               double *, double *);
int o1_fwd(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
           int, int, int, int, const double *, const double *, const double *, const double *,
           const double *, const double *, const double *, const double *, const double *,
           const double *, const double *, const double *, const double *, const double *,
           const double *, const double *, double *, double *);
int o1_set_skip(uint64_t);

static uint64_t st = 88172645463325252ull;
static double rnd(void) {   /* xorshift64, uniform in [-1, 1) */
    st ^= st << 13; st ^= st >> 7; st ^= st << 17;
    return (double)(st >> 11) / 4503599627370496.0 - 1.0;
}
static double *arr(int64_t n) {
    double *p = malloc(sizeof(double) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) p[i] = rnd();
    return p;
}

static int run(int64_t B, int64_t S, int64_t H, int64_t G, int64_t R, int64_t N, int64_t P,
               int64_t C, int64_t W, int mode, int red, int hz, int hd) {
    const int64_t nc = (S + C - 1) / C;
    double *dout = arr(red ? B * S * H * P : B * S * R * H * P);
    double *q = arr(B * S * R * G * N), *k = arr(B * S * R * G * N), *v = arr(B * S * H * P);
    double *qb = arr(H * R * N), *kb = arr(H * R * N), *mv = arr(H * R * P);
    double *mo = red ? arr(H * R * P) : NULL;
    double *z = hz ? arr(B * S * H * P) : NULL, *mz = hz ? arr(H * R * P) : NULL;
    double *ang = arr(B * S * H * W), *cs = arr(B * H * S), *rev = arr(B * H * S);
    double *dt = arr(B * H * S), *trap = arr(B * H * S), *d = hd ? arr(H) : NULL;
    double *seg = arr(B * H * nc * C * C);
    double *dmo = red ? arr(B * H * R * P) : NULL, *dmz = hz ? arr(B * H * R * P) : NULL;
    double *states = arr(B * H * nc * N * P), *dz = hz ? arr(B * S * H * P) : NULL;
    double *qk = arr(B * H * S * R * R);
    double *o = arr(red ? B * S * H * P : B * S * R * H * P);
    int rc = o1_bwd_fwd(B, S, H, G, R, N, P, C, W, mode, red, hz, hd, dout, q, k, v, qb, kb, mv, mo,
                        z, mz, ang, cs, rev, dt, trap, d, seg, dmo, states, dz, dmz, qk);
    rc |= o1_fwd(B, S, H, G, R, N, P, C, W, mode, red, hz, hd, q, k, v, qb, kb, mv, mo, z, mz, ang,
                 cs, rev, dt, trap, d, seg, o, states);
    double s = 0.0;
    for (int64_t i = 0; i < B * H * nc * N * P; ++i) s += states[i];
    for (int64_t i = 0; i < B * H * S * R * R; ++i) s += qk[i];
    free(dout); free(q); free(k); free(v); free(qb); free(kb); free(mv); free(mo); free(z); free(mz);
    free(ang); free(cs); free(rev); free(dt); free(trap); free(d); free(seg); free(dmo); free(dmz);
    free(states); free(dz); free(qk); free(o);
    return rc != 0 || !isfinite(s);
}

int main(void) {
    int bad = 0;
    for (int mode = 0; mode < 3; ++mode)
        for (int br = 0; br < 8; ++br) {
            bad |= run(1, 37, 2, 1, 2, 16, 8, 8, 4, mode, br & 1, (br >> 1) & 1, (br >> 2) & 1);
            bad |= run(2, 23, 4, 2, 3, 8, 12, 6, 2, mode, br & 1, (br >> 1) & 1, (br >> 2) & 1);
            bad |= run(1, 5, 1, 1, 1, 4, 4, 1, 1, mode, br & 1, (br >> 1) & 1, (br >> 2) & 1);
        }
    o1_set_skip(~0ull);   /* every rounding place off */
    bad |= run(1, 19, 2, 2, 4, 16, 16, 16, 4, 0, 1, 1, 1);
    o1_set_skip(0);
    printf(bad ? "FAIL\n" : "OK\n");
    return bad;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    drv = tmp_path / "driver.c"
    drv.write_text(DRIVER)
    exe = tmp_path / "o1_sanitized"
    # host C only: the oracle and its driver, with both sanitizers and no recovery
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           str(ROOT / "oracle" / "o1_contract.c"), str(drv), "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0 and res.stdout.strip() == "OK", res.stdout + res.stderr
