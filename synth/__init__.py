"""Seeded synthetic inputs for the LOCKS decode path.

This package holds only input generation (random keys, values, queries, block
tables) and none of the method's arithmetic.  Both the CPU oracle and the HIP
path consume what it produces; they never generate inputs themselves.

Recipe (one KV head of one page; d = head dim, B = 16 tokens, r = 8):
  centroid  c ~ N(0, I_d)
  u_1..u_8  a fresh Haar-random orthonormal set per page
  a_ik ~ N(0, 1/k)            (second argument read as a variance)
  noise ~ N(0, 0.05 I_d)      (variance)
  key_i = c + sum_k a_ik u_k + noise_i
  values ~ N(0, 1), queries ~ N(0, 1)
Carrier pages: per (layer, sequence, KV head) a set of distinct pages; in each
one token's key is replaced by 3 q_h/|q_h| + noise, with q_h one of the query
heads of that KV head's group (round robin over the group).
"""

from .workloads import WORKLOADS, Workload, get_workload  # noqa: F401
