"""Host <-> device marshalling for the GPU tests (no method arithmetic)."""
import numpy as np
import torch

from tree_causal_draft_parent_amd import synth

DEV = "cuda:0"


def dev_tensor(a: np.ndarray, dtype: str = None) -> torch.Tensor:
    """Upload a generated array; bf16 arrive as uint16 bit patterns."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def upload_attn(inp):
    dt = inp["dtype"]
    kv = None if inp.get("kv_dtype") == "fp8" else dt      # FP8 caches travel as raw bytes
    return dict(q=dev_tensor(inp["q"], dt), k_tree=dev_tensor(inp["k_tree"], dt),
                v_tree=dev_tensor(inp["v_tree"], dt), k_cache=dev_tensor(inp["k_cache"], kv),
                v_cache=dev_tensor(inp["v_cache"], kv), parent=dev_tensor(inp["parent"]),
                block_table=dev_tensor(inp["block_table"]))


def say(msg: str):
    print(msg, flush=True)
