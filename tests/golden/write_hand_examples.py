"""Writes hand_examples.json: closed-form decode-attention examples.

Every expected number is derived by hand from the definition of attention and
evaluated here with the math module only (ln 3, sigmoid(2), ...).  No
implementation of attention, oracle or kernel, is called.
Run from the repository root:  python tests/golden/write_hand_examples.py
"""
import json
import math
import pathlib

LN2, LN3, LN4 = math.log(2.0), math.log(3.0), math.log(4.0)

EXAMPLES = {
    "_about": ("Hand-worked decode-attention examples. Every expected value below is derived on paper "
               "from the definition of attention (scores = scale*<q,k_j>, softmax over the valid rows, "
               "weighted sum of the value rows; lse = natural log of the softmax denominator) and is "
               "stored here as a closed-form number. None of them comes from any implementation."),
    "examples": [
        {"name": "two_keys_one_to_three",
         "cite": "Flash Attention memory-traffic page (shop.zimaspace.com), section on standard attention: scores from q and K, normalised, combined with V",
         "derivation": "scores 0 and ln 3 -> weights 1/4, 3/4 -> out = [4/4, 3*8/4] = [1, 6]; lse = ln(1+3) = ln 4",
         "scale": 1.0, "q": [[[1.0, 0.0]]], "k": [[[[0.0, 0.0], [LN3, 0.0]]]],
         "v": [[[[4.0, 0.0], [0.0, 8.0]]]], "lens": [2],
         "out": [[[1.0, 6.0]]], "lse": [[LN4]]},
        {"name": "equal_scores_three_keys",
         "cite": "same section: equal scores give equal weights",
         "derivation": "all three scores equal 2 -> weights 1/3 each -> out = mean of V rows = [2, 2]; lse = 2 + ln 3",
         "scale": 1.0, "q": [[[2.0, 1.0]]], "k": [[[[1.0, 0.0], [1.0, 0.0], [0.0, 2.0]]]],
         "v": [[[[3.0, 0.0], [0.0, 3.0], [3.0, 3.0]]]], "lens": [3],
         "out": [[[2.0, 2.0]]], "lse": [[2.0 + LN3]]},
        {"name": "default_scale_sigmoid",
         "cite": "same section; scale 1/sqrt(D) is the reading taken for the unstated temperature",
         "derivation": "D=4, scale=1/2; raw dots 0 and 4 -> scores 0 and 2 -> weight of row 1 is sigmoid(2) -> every coordinate of out = e^2/(1+e^2); lse = ln(1+e^2)",
         "scale": None, "q": [[[1.0, 1.0, 1.0, 1.0]]], "k": [[[[0.0, 0.0, 0.0, 0.0], [1.0, 1.0, 1.0, 1.0]]]],
         "v": [[[[0.0, 0.0, 0.0, 0.0], [1.0, 1.0, 1.0, 1.0]]]], "lens": [2],
         "out": [[[1.0 / (1.0 + math.exp(-2.0))] * 4]], "lse": [[math.log1p(math.exp(2.0))]]},
        {"name": "gqa_contiguous_groups",
         "cite": "bifurcated-attention page (linnk.ai), section Tilastot: query heads share KV heads in groups; contiguous grouping is the reading taken",
         "derivation": "Hq=4, Hkv=2: heads 0,1 read KV head 0 (uniform over V=1,3 -> 2), heads 2,3 read KV head 1 (uniform over V=10,20 -> 15); lse = ln 2 for every head (all scores 0)",
         "scale": 1.0, "q": [[[1.0], [1.0], [1.0], [1.0]]],
         "k": [[[[0.0], [0.0]], [[0.0], [0.0]]]], "v": [[[[1.0], [3.0]], [[10.0], [20.0]]]], "lens": [2],
         "out": [[[2.0], [2.0], [15.0], [15.0]]], "lse": [[LN2] * 4]},
        {"name": "ragged_batch_ignores_padding",
         "cite": "Flash-Decoding page (slavadubrov.com), section on why decoding needs another schedule: each sequence attends over its own cached history only",
         "derivation": "sequence 0 has 1 valid row (out = that V row = [5]); sequence 1 has 2 valid rows with scores 0, ln 3 -> out = (1*1 + 3*9)/4 = 7; padding rows hold 1e30 and must not matter",
         "scale": 1.0, "q": [[[1.0]], [[1.0]]],
         "k": [[[[0.0], [1e30]]], [[[0.0], [LN3]]]], "v": [[[[5.0], [1e30]]], [[[1.0], [9.0]]]],
         "lens": [1, 2], "out": [[[5.0]], [[7.0]]], "lse": [[0.0], [LN4]]},
    ],
    "combine_examples": [
        {"name": "two_pieces_and_an_empty_one",
         "cite": "Flash-Decoding page, section on why decoding needs another schedule: pieces yield (partial output, log-sum-exp) and a reduction renormalises them",
         "derivation": "piece weights exp(0):exp(ln 3):0 = 1:3:0 -> out = (1*2 + 3*6)/4 = 5; lse = ln(1 + 3) = ln 4",
         "o_part": [[[2.0]], [[6.0]], [[0.0]]], "lse_part": [[0.0], [LN3], [None]],
         "out": [[5.0]], "lse": [LN4]},
    ],
    "paged_examples": [
        {"name": "reversed_pages_exclude_the_tail",
         "cite": "memory-wall page (gyaansetu.com), section on fighting the memory wall, PagedAttention paragraph: cache rows in fixed-size blocks reached through an indirection table",
         "derivation": "page size 2. Sequence 0 uses pages [1, 0] and 3 rows: page1 row0 (K 0, V 6), page1 row1 (K ln 2, V 0), page0 row0 (K ln 3, V 2); page0 row1 (K 100) lies past the length. Weights 1:2:3 -> out = (6 + 0 + 3*2)/6 = 2, lse = ln 6. Sequence 1 uses page 2 and 1 row (K 5, V 50) -> out 50, lse 5",
         "scale": 1.0, "q": [[[1.0]], [[1.0]]], "page_size": 2,
         "k_pages": [[[[LN3], [100.0]]], [[[0.0], [LN2]]], [[[5.0], [5.0]]]],
         "v_pages": [[[[2.0], [1000.0]]], [[[6.0], [0.0]]], [[[50.0], [50.0]]]],
         "block_table": [[1, 0], [2, 1]], "lens": [3, 1],
         "out": [[[2.0]], [[50.0]]], "lse": [[math.log(6.0)], [5.0]]},
    ],
    "fp8kv_examples": [
        {"name": "e4m3_codes_with_head_scales",
         "cite": "memory-wall page (gyaansetu.com), section on fighting the memory wall, quantisation paragraph: fewer bits per stored value; E4M3 codes as defined by the OCP 8-bit floating-point specification (bias 7)",
         "derivation": "K codes 0x00 = 0 and 0x38 = 1.0 with k_scale ln 3 -> scores 0 and ln 3 -> weights 1:3. V codes 0x40 = 2.0 and 0x48 = 4.0 with v_scale 1/2 -> values 1 and 2 -> out = (1 + 3*2)/4 = 7/4; lse = ln 4",
         "scale": 1.0, "q": [[[1.0]]], "k_bits": [[[[0], [56]]]], "v_bits": [[[[64], [72]]]],
         "k_scale": [LN3], "v_scale": [0.5], "lens": [2],
         "out": [[[1.75]]], "lse": [[LN4]]},
    ],
    "bifurcated_examples": [
        {"name": "context_plus_own_decode_rows",
         "cite": "bifurcated-attention page (linnk.ai), section Tiivistelmä: the context part and the decode part together give exact attention",
         "derivation": "context row K=0, V=1 shared. Sample 0 adds its own row K=0, V=3 -> uniform over two rows -> 2, lse ln 2. Sample 1 has no decode rows -> out 1, lse 0",
         "scale": 1.0, "q": [[[1.0]], [[1.0]]], "k_ctx": [[[0.0]]], "v_ctx": [[[1.0]]],
         "k_dec": [[[[0.0]]], [[[7.0]]]], "v_dec": [[[[3.0]]], [[[100.0]]]], "dec_lens": [1, 0],
         "out": [[[2.0]], [[1.0]]], "lse": [[LN2], [0.0]]},
    ],
}

if __name__ == "__main__":
    path = pathlib.Path(__file__).with_name("hand_examples.json")
    path.write_text(json.dumps(EXAMPLES, indent=1) + "\n")
    print("wrote", path)
