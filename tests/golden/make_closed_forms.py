"""Write closed_forms.json: tiny MLA decode cases whose answers are closed forms.

The pages print no worked example with numbers, so these fixtures are derived by
hand from the definition (TileLang MLA guide, "参考实现与正确性验证": softmax of
the scaled [q ‖ q_pe]·[kv ‖ k_pe] scores, weighted sum of the latent rows) and
from the combine rule ("Combine Kernel" section: anchor at the largest base-2
lse, weight each partial by 2^(lse_k - lse_total)).  Expected values are
evaluated here with the ``math`` module only; nothing is computed by the
oracle or by the GPU library.

Sparse encoding: ``q`` and ``rows`` list ``[d, value]`` pairs with d in 0..575
(d >= 512 is the RoPE part); all other entries are zero.  With
softmax_scale = 1/8 and q[d=0] = 8, the score of row j is exactly row_j[0].
"""
import json
import math
import os

E = math.e


def main():
    cases = []
    # Scores 0 and 1: weights 1/(1+e), e/(1+e).
    w0, w1 = 1 / (1 + E), E / (1 + E)
    two_rows = dict(
        heads=1, dtype="f16", softmax_scale=0.125,
        q=[[[0, 8.0]]],
        rows=[[[0, 0.0], [1, 0.5]], [[0, 1.0], [1, -2.0]]],
        expect=[dict(lse=math.log(1 + E), out=[[0, w1], [1, 0.5 * w0 - 2.0 * w1]])],
    )
    cases.append(dict(name="two_rows_scores_0_1", **two_rows))
    # Same rows reached through a reversed block_table with one-row pages.
    cases.append(dict(name="two_rows_paged_reversed", paged=True, page_block_size=1,
                      block_table=[1, 0], **two_rows))
    # One row: out is its latent part, lse its score (0.125 * 0.25 * 2 = 1/16).
    cases.append(dict(
        name="seqlen_one", heads=1, dtype="f16", softmax_scale=0.125,
        q=[[[520, 0.25]]],
        rows=[[[0, 3.0], [5, -1.5], [520, 2.0]]],
        expect=[dict(lse=0.0625, out=[[0, 3.0], [5, -1.5]])],
    ))
    # q = 0: all scores 0, out = mean of rows, lse = ln 3; two heads.
    cases.append(dict(
        name="equal_scores_mean", heads=2, dtype="f16", softmax_scale=0.125,
        q=[[], []],
        rows=[[[0, 1.0]], [[0, 2.0], [7, 3.0]], [[0, -6.0]]],
        expect=[dict(lse=math.log(3), out=[[0, -1.0], [7, 1.0]])] * 2,
    ))
    # Scores 0, 1, 2 cut into splits of rows {0,1} and {2} (one-row blocks).
    den = 1 + E + E * E
    cases.append(dict(
        name="three_rows_two_splits", heads=1, dtype="f16", softmax_scale=0.125,
        splits=2, block_rows=1,
        q=[[[0, 8.0]]],
        rows=[[[0, 0.0]], [[0, 1.0]], [[0, 2.0]]],
        expect=[dict(lse=math.log(den), out=[[0, (E + 2 * E * E) / den]])],
    ))
    combine_cases = [
        # lse2 1 and 3: total log2(10), weights 0.2 and 0.8.
        dict(name="combine_two", partial_out=[[1.0, 0.0], [0.0, 1.0]], partial_lse2=[1.0, 3.0],
             out=[0.2, 0.8], lse=math.log(10.0)),
        # An empty split (lse2 = -inf) contributes nothing.
        dict(name="combine_with_empty", partial_out=[[5.0, 5.0], [0.5, -0.25]],
             partial_lse2=[-math.inf, 2.0], out=[0.5, -0.25], lse=2.0 * math.log(2.0)),
        # All empty: zero output and -inf lse.
        dict(name="combine_all_empty", partial_out=[[0.0, 0.0], [0.0, 0.0]],
             partial_lse2=[-math.inf, -math.inf], out=[0.0, 0.0], lse=-math.inf),
    ]
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "closed_forms.json")
    with open(path, "w") as f:
        json.dump(dict(source="hand-derived closed forms; see make_closed_forms.py",
                       cases=cases, combine_cases=combine_cases), f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
