"""Writes attention_worked_examples.json: tiny attention cases worked out by hand.

Every expected value is derived in its "derivation" field from the definition
of attention alone (scores, softmax, weighted sum of values, paged addressing)
and written here with math.log only: no oracle and no library code runs.
The pages print no numeric attention output, so these closed forms stand in
for a worked example.
"""
import json
import math
import os

L3 = math.log(3.0)
CITATION = ("the-ai.news, 'Snelle attention-kernels en operatorfusie versnellen AI-modellen', section "
            "'FlashAttention-type aandacht en gepagineerde aandacht' (score matrix per head, softmax "
            "statistics, output accumulated from values; paged positions translated through a block "
            "table, 16-token blocks in the vLLM example). Expected values below are worked out by hand "
            "from that definition; none comes from any implementation.")

CASES = [
    {"name": "two_keys_quarter_three_quarters", "kind": "prefill",
     "derivation": "scores are 0 and ln3, so the softmax weights are 1/4 and 3/4; O = v0/4 + 3 v1/4 = [1, 6]; "
                   "lse = ln(1 + 3) = ln 4",
     "scale": 1.0, "causal": False, "seq_lens": None,
     "q": [[[[L3]]]], "k": [[[[0.0], [1.0]]]], "v": [[[[4.0, 0.0], [0.0, 8.0]]]],
     "o": [[[[1.0, 6.0]]]], "lse": [[[math.log(4.0)]]]},
    {"name": "causal_scale0_running_mean", "kind": "prefill",
     "derivation": "scale 0 makes every visible score 0: row i averages v_0..v_i (causal, diagonal included); "
                   "lse_i = ln(i+1)",
     "scale": 0.0, "causal": True, "seq_lens": None,
     "q": [[[[1.0], [2.0], [3.0]]]], "k": [[[[5.0], [-1.0], [2.0]]]], "v": [[[[3.0], [6.0], [9.0]]]],
     "o": [[[[3.0], [4.5], [6.0]]]], "lse": [[[0.0, math.log(2.0), math.log(3.0)]]]},
    {"name": "causal_bottom_right_tq2_tk4", "kind": "prefill",
     "derivation": "bottom-right causal alignment: query i sees keys j <= i + (Tk - Tq) = i + 2; scale 0 averages "
                   "the visible values: row 0 -> mean(2,4,6) = 4, row 1 -> mean(2,4,6,8) = 5; lse = ln 3, ln 4",
     "scale": 0.0, "causal": True, "seq_lens": None,
     "q": [[[[1.0], [1.0]]]], "k": [[[[1.0], [1.0], [1.0], [1.0]]]], "v": [[[[2.0], [4.0], [6.0], [8.0]]]],
     "o": [[[[4.0], [5.0]]]], "lse": [[[math.log(3.0), math.log(4.0)]]]},
    {"name": "ragged_scale0_padding_rows", "kind": "prefill",
     "derivation": "lengths [2, 3] on a padded length of 3: sequence 0 averages v_0, v_1 = (1+3)/2 = 2 for rows 0 "
                   "and 1; its row 2 is padding (O = 0, lse = -inf); sequence 1 averages all three "
                   "(10+20+60)/3 = 30; lse = ln 2 / ln 3",
     "scale": 0.0, "causal": False, "seq_lens": [2, 3],
     "q": [[[[1.0], [1.0], [1.0]]], [[[1.0], [1.0], [1.0]]]],
     "k": [[[[1.0], [1.0], [1.0]]], [[[1.0], [1.0], [1.0]]]],
     "v": [[[[1.0], [3.0], [100.0]]], [[[10.0], [20.0], [60.0]]]],
     "o": [[[[2.0], [2.0], [0.0]]], [[[30.0], [30.0], [30.0]]]],
     "lse": [[[math.log(2.0), math.log(2.0), "-inf"]], [[math.log(3.0)] * 3]]},
    {"name": "gqa_consecutive_heads_share_kv", "kind": "prefill",
     "derivation": "one key per kv head, so each query head returns its kv head's single value: heads 0,1 read kv "
                   "head 0 (value 1), heads 2,3 read kv head 1 (value 2); lse = scale*q.k = 3 and 5",
     "scale": 1.0, "causal": False, "seq_lens": None,
     "q": [[[[1.0]], [[1.0]], [[1.0]], [[1.0]]]], "k": [[[[3.0]], [[5.0]]]], "v": [[[[1.0]], [[2.0]]]],
     "o": [[[[1.0]], [[1.0]], [[2.0]], [[2.0]]]], "lse": [[[3.0], [3.0], [5.0], [5.0]]]},
    {"name": "large_scores_need_max_subtraction", "kind": "prefill",
     "derivation": "two equal scores of 1000 (exp would overflow without subtracting the row max): O = mean(v) = 5, "
                   "lse = 1000 + ln 2",
     "scale": 1.0, "causal": False, "seq_lens": None,
     "q": [[[[1000.0]]]], "k": [[[[1.0], [1.0]]]], "v": [[[[4.0], [6.0]]]],
     "o": [[[[5.0]]]], "lse": [[[1000.0 + math.log(2.0)]]]},
    {"name": "paged_two_slot_blocks", "kind": "decode",
     "derivation": "2-slot blocks, context 3, table [2, 0]: positions 0,1 live in block 2 slots 0,1 (values 7, 11), "
                   "position 2 in block 0 slot 0 (value 3); block 1 and block 0 slot 1 are never read; scale 0 "
                   "averages (7+11+3)/3 = 7; lse = ln 3",
     "scale": 0.0, "ctx_lens": [3], "block_table": [[2, 0]],
     "q": [[[1.0]]],
     "k_cache": [[[[1.0], [1.0]]], [[[1.0], [1.0]]], [[[1.0], [1.0]]]],
     "v_cache": [[[[3.0], [999.0]]], [[[-50.0], [-60.0]]], [[[7.0], [11.0]]]],
     "o": [[[7.0]]], "lse": [[math.log(3.0)]]},
]

if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "attention_worked_examples.json")
    with open(out, "w") as f:
        json.dump({"citation": CITATION, "cases": CASES}, f, indent=1)
    print("wrote", out)
