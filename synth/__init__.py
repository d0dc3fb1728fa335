"""Seeded synthetic inputs for the LOCKS decode path.

This module only draws random tensors with the shapes and structure of the
workloads (Llama-3.1-8B-shaped paged KV: d = 128, B = 16, 8 KV heads, GQA
group 4). It holds none of the method's arithmetic and is the only code shared
by the oracle side and the GPU side of the tests and the benchmark.

Key generator for page j (every page has its own rank-8 structure):
    k_i = mu_j + U_j diag(3, 2.5, 2, 1.6, 1.3, 1, 0.8, 0.6) z_i + 0.05 eps_i
with mu_j ~ N(0, I_d), U_j a random orthonormal d x 8 basis (modified
Gram-Schmidt of a Gaussian matrix), z_i ~ N(0, I_8), eps_i ~ N(0, I_d).
A planted needle token has key 6 q_dir / |q_dir|. Queries of a GQA group are
q_g = q_dir + 0.3 N(0, I_d) with one q_dir ~ N(0, I_d) per (layer, KV head).
Values ~ N(0, 1). Every tensor is rounded to bf16 (round to nearest even).
"""
from .locks_inputs import *  # noqa: F401,F403
