"""Planted mistakes in copies of the CPU oracle must each fail a pin.

Every mutation below is a plausible slip (a dropped term, a wrong sign or
index, a wrong face value, a wrong scalar in the Krylov step).  The copy is
compiled on the CPU with the same flags as the oracle and the full pin set
of oracle_pins.py is run against it; the test passes only if some pin fails.
"""
import os

import pytest

import oracle
import oracle_pins as P

MUTATIONS = {
    "dot_no_compensation": ("    return s + c;\n}", "    (void)c;\n    return s;\n}"),
    "dot_kahan_branch": ("        if (fabs(s) >= fabs(t))\n            c += (s - u) + t;\n        else\n            c += (t - u) + s;",
                         "        c += (s - u) + t;"),
    "dot_wrong_operand": ("        double t = a[l] * b[l];\n        double u = s + t;", "        double t = a[l] * a[l];\n        double u = s + t;"),
    "stencil_drop_ym": ("acc += face_ym(nx, ny, ah, i, j) * (u - x[at(nx, nz, i, jm, k)]);", ""),
    "stencil_vertical_sign": ("acc += az[k + 1] * (u - x[at(nx, nz, i, j, k + 1)]);",
                              "acc -= az[k + 1] * (u - x[at(nx, nz, i, j, k + 1)]);"),
    "stencil_no_wrap": ("int ip = (i + 1) % nx, im = (i + nx - 1) % nx;",
                        "int ip = (i + 1 < nx) ? i + 1 : i, im = (i + nx - 1) % nx;"),
    "stencil_face_index": ("acc += az[k + 1] * (u - x[at(nx, nz, i, j, k + 1)]);",
                           "acc += az[k] * (u - x[at(nx, nz, i, j, k + 1)]);"),
    "face_not_mean": ("return 0.5 * (ah[(size_t)j * nx + i] + ah[(size_t)j * nx + ip]);",
                      "(void)ip; return ah[(size_t)j * nx + i];"),
    "precond_drop_alphaT": ("double aT = orc_alpha_T(nx, ny, ah, i, j);", "double aT = 0.0;"),
    "precond_back_sign": ("z[at(nx, nz, i, j, k)] -= gam[k + 1] * z[at(nx, nz, i, j, k + 1)];",
                          "z[at(nx, nz, i, j, k)] += gam[k + 1] * z[at(nx, nz, i, j, k + 1)];"),
    "precond_upper_face": ("double up = (k < nz - 1) ? az[k + 1] : 0.0;",
                           "double up = (k < nz - 1) ? az[k] : 0.0;"),
    "pcg_beta_inverted": ("double beta = rho_new / rho;", "double beta = rho / rho_new;"),
    "pcg_alpha_wrong_dot": ("double alpha = rho / sigma;", "double alpha = rho / orc_dot(n, q, q);"),
    "pcg_x_sign": ("for (size_t l = 0; l < n; ++l) x[l] += alpha * p[l];",
                   "for (size_t l = 0; l < n; ++l) x[l] -= alpha * p[l];"),
    "pcg_r_uses_p": ("for (size_t l = 0; l < n; ++l) r[l] -= alpha * q[l];",
                     "for (size_t l = 0; l < n; ++l) r[l] -= alpha * p[l];"),
    "pcg_extra_step": ("for (int k = 1; k <= maxit; ++k) {", "for (int k = 1; k <= maxit + 1; ++k) {"),
    "pcg_p_no_beta": ("for (size_t l = 0; l < n; ++l) p[l] = z[l] + beta * p[l];",
                      "for (size_t l = 0; l < n; ++l) p[l] = z[l];"),
    "pcg_residual_sign": ("r[l] = b[l] - q[l];", "r[l] = b[l] + q[l];"),
    "f32_stencil_drop_xm": ("acc += face_f32(ah, c, (size_t)j * nx + im) * (u - x[at(nx, nz, im, j, k)]);", ""),
    "f32_precond_back_sign": ("z[at(nx, nz, i, j, k)] -= gam[k + 1] * z[at(nx, nz, i, j, k + 1)];\n        }\n    free(gam);\n    return status;\n}\n\n/* <a,b> of binary32",
                              "z[at(nx, nz, i, j, k)] += gam[k + 1] * z[at(nx, nz, i, j, k + 1)];\n        }\n    free(gam);\n    return status;\n}\n\n/* <a,b> of binary32"),
    "f32_pcg_beta_inverted": ("const float beta = (float)(rho_new / rho);", "const float beta = (float)(rho / rho_new);"),
    "mixed_stale_residual": ("        for (size_t l = 0; l < n; ++l) r32[l] = (float)r[l];", ""),
    "gen_drop_d": ("acc += d[k] * hor;", "acc += hor;"),
    "gen_x_edge_index": ("hor += ax[(size_t)j * nx + im] * (u - x[at(nx, nz, im, j, k)]);",
                         "hor += ax[(size_t)j * nx + i] * (u - x[at(nx, nz, im, j, k)]);"),
    "gen_precond_no_area": ("double sub = -T * beta[k];", "double sub = -beta[k];"),
    "gen_alphaT_missing_edge": ("return ax[(size_t)j * nx + i] + ax[(size_t)j * nx + im]",
                                "return ax[(size_t)j * nx + i] + 0.0 * ax[(size_t)j * nx + im]"),
    "mg_coarse_edge_index": ("sx += ax[(size_t)(fy * J + b) * nx + (fx * I + fx - 1)];",
                             "sx += ax[(size_t)(fy * J + b) * nx + (fx * I)];"),
    "mg_self_edge_kept": ("cax[(size_t)J * ncx + I] = (ncx == 1) ? 0.0 : sx;", "cax[(size_t)J * ncx + I] = sx;"),
    "mg_area_not_summed": ("sa += area[(size_t)(fy * J + b) * nx + (fx * I + a)];",
                           "sa = area[(size_t)(fy * J + b) * nx + (fx * I + a)];"),
    "mg_restrict_average": ("C->f[at(C->nx, nz, i / fx, j / fy, k)] += L->t[at(nx, nz, i, j, k)];",
                            "C->f[at(C->nx, nz, i / fx, j / fy, k)] += 0.25 * L->t[at(nx, nz, i, j, k)];"),
    "mg_prolong_wrong_parent": ("+= C->z[at(C->nx, nz, i / fx, j / fy, k)];",
                                "+= C->z[at(C->nx, nz, (i / fx + 1) % C->nx, j / fy, k)];"),
    "mg_no_damping": ("z[l] += omega * L->y[l];", "z[l] += L->y[l];"),
    "mg_no_post_smooth": ("""        z[at(nx, nz, i, j, k)] += C->z[at(C->nx, nz, i / fx, j / fy, k)];
    for (int s = 0; s < nu; ++s)""", """        z[at(nx, nz, i, j, k)] += C->z[at(C->nx, nz, i / fx, j / fy, k)];
    for (int s = 0; s < 0; ++s)"""),
    "mg_coarsest_not_exact": ("        if (nx * ny == 1)\n            return orc_precond_gen(",
                              "        if (nx * ny == 0)\n            return orc_precond_gen("),
    "mg_cheb_momentum_sign": ("znew[l] = (z[l] + (rho * rho_prev) * (z[l] - zold[l]))",
                              "znew[l] = (z[l] - (rho * rho_prev) * (z[l] - zold[l]))"),
    "mg_cheb_rho_recurrence": ("const double rho = 1.0 / (2.0 * s - rho_prev);",
                               "const double rho = 1.0 / (2.0 * s + rho_prev);"),
    "mg_cheb_first_step_unscaled": ("        z[l] = L->y[l] / theta;", "        z[l] = L->y[l];"),
    "mg_cheb_stale_residual": ("            L->t[l] = f[l] - L->t[l];\n        if (orc_precond_gen(L->nx, L->ny, nz, a, d, beta, L->area, L->ax, L->ay, L->t, L->y) != ORC_OK) {",
                               "            L->t[l] = f[l];\n        if (orc_precond_gen(L->nx, L->ny, nz, a, d, beta, L->area, L->ax, L->ay, L->t, L->y) != ORC_OK) {"),
    "mg_cheb_interval_width": ("theta = 0.5 * (hi + lo), delta = 0.5 * (hi - lo)", "theta = 0.5 * (hi + lo), delta = (hi - lo)"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    mutated = src.replace(old, new, 1)
    path = os.path.join(tmp_path, "mut.c")
    with open(path, "w") as f:
        f.write(mutated)
    lib = oracle.compile_source(path, os.path.join(tmp_path, "libmut.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, FloatingPointError, ValueError, Exception) as e:  # noqa: B014
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {name}"
