"""The pages' parameter, byte and time arithmetic for expert parallelism.

Each function states one quantity the pages compute; the printed values are
pinned in tests/golden/pages_arithmetic.json.
* "Expert Parallel and All-to-All Backends" (aiinfrainterviews), "Why expert
  parallelism exists": an expert is gate, up and down matrices of H x I; the
  per-token expert read is k experts; the all-to-all moves hidden x bytes x k
  per token per direction.
* "Your expert-parallel deployment is slower..." (aiinfrainterviews Q&A),
  "A strong answer": two all-to-alls per sparse layer, time = bytes / link rate,
  and the imbalance arithmetic of a synchronous step.
* "6.4 Data parallelism and expert parallelism" (infra-guide), sections 2.1,
  2.3, 3.2 and 5.3: DeepSeek-V3 expert size and share, per-card expert memory,
  FP8 dispatch / BF16 combine bytes, redundant-expert memory and slots.
"""
from __future__ import annotations


def expert_params(H: int, I: int) -> int:
    """Parameters of one SwiGLU expert (gate and up H x I, down I x H)."""
    return 3 * H * I


def expert_bytes(H: int, I: int, bytes_per_param: float) -> float:
    return expert_params(H, I) * bytes_per_param


def expert_read_per_token(k: int, H: int, I: int, bytes_per_param: float):
    """Expert weight bytes one token reads across the system (k experts)."""
    return k * expert_bytes(H, I, bytes_per_param)


def a2a_bytes_per_token(H: int, bytes_per_elem: float, k: int) -> float:
    """All-to-all volume of one token in one direction: k copies of H."""
    return H * bytes_per_elem * k


def a2a_bytes_per_token_all_layers(H, bytes_per_elem, k, layers) -> float:
    """Dispatch plus combine over every sparse layer."""
    return 2 * layers * a2a_bytes_per_token(H, bytes_per_elem, k)


def transfer_seconds(nbytes: float, bytes_per_second: float) -> float:
    return nbytes / bytes_per_second


def nic_bytes_per_second(gbit_per_second: float) -> float:
    return gbit_per_second * 1e9 / 8.0


def read_to_comm_ratio(read_bytes: float, comm_bytes: float) -> float:
    return read_bytes / comm_bytes


def idle_fraction(busiest_over_mean: float) -> float:
    """Share of a synchronous phase the other ranks wait for the busiest."""
    return 1.0 - 1.0 / busiest_over_mean


def step_growth(moe_fraction: float, busiest_over_mean: float) -> float:
    """Relative growth of a step whose MoE share slows by the imbalance."""
    return moe_fraction * busiest_over_mean + (1.0 - moe_fraction) - 1.0


def routed_params(layers: int, experts: int, H: int, I: int) -> int:
    return layers * experts * expert_params(H, I)


def per_card_expert_bytes(layers, experts, ep, H, I, bytes_per_param):
    return layers * (experts // ep) * expert_params(H, I) * bytes_per_param


def redundant_expert_bytes(layers, H, I, bytes_per_param) -> float:
    """Memory of one redundant expert replicated in every MoE layer."""
    return layers * expert_params(H, I) * bytes_per_param


def experts_per_card(experts: int, redundant: int, ep: int) -> int:
    return (experts + redundant) // ep


def dispatch_combine_saving(k, H, dispatch_bytes, combine_bytes,
                            base_bytes=2) -> float:
    """Fraction of round-trip bytes saved versus base_bytes both ways."""
    base = 2 * k * H * base_bytes
    return 1.0 - (k * H * dispatch_bytes + k * H * combine_bytes) / base
