"""Benchmark placeholder: model functions only (the runner follows)."""


def gemm_flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def naive_model_bytes(M: int, N: int, K: int) -> int:
    return 8 * M * N * K


def tiled_model_bytes(M: int, N: int, K: int, BM: int, BN: int) -> int:
    tiles = -(-M // BM) * -(-N // BN)
    return 4 * K * tiles * (BM + BN)
