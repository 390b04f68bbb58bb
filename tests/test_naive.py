"""GPU parity of the unfused three-kernel baseline (attn_fwd_naive) with the
fp64 oracle: the same results as the fused path, through materialised S and P."""
import pytest

from parity_util import full_case
from scaled_dot_product_flashattention_amd.inputs import WORKLOADS

pytestmark = pytest.mark.gpu

W = WORKLOADS
CASES = {
    "tiny_fp32": W["tiny_fp32"],
    "medium_bf16": W["medium_bf16"].replace(H=2, Sq=700, Sk=900),
    "long_causal_bf16": W["long_causal_bf16"].replace(B=1, H=2, Sq=600, Sk=600),
    "bert_pad_fp16": W["bert_pad_fp16"].replace(B=4, H=2),
    "ragged_f32_d128": W["tiny_fp32"].replace(name="ragged", B=2, H=1, Sq=77, Sk=130, d=128,
                                               layout="bshd", causal=True),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_naive_matches_oracle(name):
    full_case(CASES[name], path="naive", poison=CASES[name].kv_len_range is not None)
