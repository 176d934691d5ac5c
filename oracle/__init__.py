"""CPU oracle for the MoE token-routing and dispatch path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or
links this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it. It shares no code, table or
helper with the HIP library.

Every function is a plain, slow, obviously correct definition written from
three web pages on the subject (``oracle.eg`` holds the s-EG expert
placement of the "Speculative MoE" notes, sections 3.2 and 4.2;
``oracle.estfit`` the estimator fit of "Speculating Experts", item 2.C;
``oracle.prefetch`` the expert prefetch plan of "Speculating Experts",
items 1, 2 and 4):

* "Speculative MoE" notes (research-notes-783.pages.dev/p/speculative-moe/):
  route prediction tables (section 4.1), the shuffled reduce-scatter SRS and
  its inverse SAG (section 3.1), expert dispatch/combine (section 1), local
  activation rate (section 7 glossary);
* "Speculating Experts Accelerates Inference for Mixture-of-Experts"
  (gist.science/ko/paper/2603.19289): quasi-hidden state q_l and the
  lightweight estimator (technical summary, items 2.A and 2.C), hit rate
  (item 4);
* "Federation of Experts (FoE)" (aitrends.kr/articles/58129): grouped
  top-k/H routing and the locality rho formulas (grouped MoE block and
  per-layer comparison paragraphs).

Floating point is float64 unless the step's output is itself a quantised code
decided by float arithmetic (the SRS bf16 sum, the table builder's argmax);
those take the kernel's float32 precision and order, as stated per function.

Parity status per function (what pins it) is listed in ``PINS``.
"""

from .bf16 import bf16_to_f64, round_bf16, f32_to_bf16
from .route import (
    route_predict,
    srs_shuffle,
    route_gate,
    route_topk,
    lar_count,
    moe_permute,
    moe_combine,
    route_qhidden,
    gelu_erf,
    route_estimator,
    hit_count,
    route_lut_build,
)
from .pipeline import route_pass, foe_pass, predictor_layer_pass

PINS = {
    "round_bf16": "torch CPU float32->bf16 conversion; hand-derived tie cases",
    "route_predict": "np.take when no fallback; 2-gram table when all fall back; dict brute force",
    "srs_shuffle": "bucket-loop brute force; P=1 pure permutation; G=1 pure reduce; "
                   "P=2 exact rational rounding",
    "route_gate": "one-hot operand closed forms; integer-valued exact products",
    "route_topk": "all-subsets brute force; H=1 grouped == plain; K=E permutation; "
                  "planted ties and signed zeros; scipy softmax",
    "lar_count": "rho_moe = 1/G and rho_foe = min(H/G, 1) under uniform routing; all-local = 1",
    "moe_permute": "bijection; counts sum to N*K; stability; list brute force",
    "moe_combine": "identity experts return the input; one-hot weights select a slot",
    "route_qhidden": "torch layer_norm in float64; mean 0 / variance s2/(s2+eps)",
    "route_estimator": "math.erf GELU; torch linear in float64",
    "hit_count": "pred == truth gives N*K; disjoint gives 0; random gives about K/E",
    "route_lut_build": "per-id brute force over cluster shares",
    "eg.splitmix64": "first three published outputs of the reference generator (seed 0)",
    "eg.coact_profile": "conservation: counts sum to n*K, rows to K*freq",
    "eg.eg_score": "G=1 gives all local; T/G <= local <= T; relabelling; planted all-local",
    "eg.eg_objective": "closed forms (all local + balanced = 0; nothing local + one full cluster)",
    "eg.eg_sample": "equal capacity always; a one-hot table is reproduced; first-draw frequencies",
    "eg.eg_update": "one elite with alpha=1 gives its one-hot; tie to lower index; incumbent kept",
    "eg.ceo_place": "finds the planted block placement (every activation local)",
    "estfit.est_gram": "Hadamard features give n*I; last row/diagonal are column sums and n",
    "estfit.est_solve": "closed form on orthogonal features; exact linear target recovered; "
                        "ridge residual identity",
    "estfit.est_weights": "transpose and bf16 rounding of the recovered weights",
    "prefetch.prefetch_plan": "hand-worked example; one token gives its predicted set; "
                              "brute-force best C-subset with the stated order",
    "prefetch.prefetch_coverage": "hand-worked example; set intersection for one token; "
                                  "covered + missed picks = n*K; prediction = truth covers all",
    "prefetch.prefetch_copy": "listed slots equal their bank rows, unlisted slots unchanged",
}
