"""Unpacks the library's quantized-operand byte layouts into the plain logical
layouts the oracle uses, following the layout description in
include/sage_mi355x.h (T = ceil(N/64), Nq = 128*ceil(N/128), G = Nq/32):

  q_i8  byte ((bh*G + g)*4096 + (kk*64 + l)*16 + i) = Q[32g + l%32][32kk + 16(l/32) + i]
  k_i8  byte ((bh*T + t)*8192 + ((half*4 + kk)*64 + l)*16 + i)
                                    = K[64t + 32half + l%32][32kk + 16(l/32) + i]
  v_fp8 byte ((bh*T + t)*8192 + ((db*2 + half)*64 + l)*16 + i)
                                    = V[64t + 32half + 8(i/4) + 4(l/32) + i%4][32db + l%32]
"""
import numpy as np


def q_logical(raw, B, H, N):
    Nq = -(-N // 128) * 128
    G = Nq // 32
    a = np.asarray(raw).reshape(B, H, G, 4, 2, 32, 16)        # b h g kk hh r i
    return a.transpose(0, 1, 2, 5, 3, 4, 6).reshape(B, H, Nq, 128)


def k_logical(raw, B, H, N):
    T = -(-N // 64)
    a = np.asarray(raw).reshape(B, H, T, 2, 4, 2, 32, 16)     # b h t half kk hh r i
    return a.transpose(0, 1, 2, 3, 6, 4, 5, 7).reshape(B, H, T * 64, 128)


def v_logical(raw, B, H, N):
    T = -(-N // 64)
    a = np.asarray(raw).reshape(B, H, T, 4, 2, 2, 32, 4, 4)   # b h t db half hh dl i4 i1
    # key = 32half + 8i4 + 4hh + i1, d = 32db + dl
    return a.transpose(0, 1, 2, 4, 7, 5, 8, 3, 6).reshape(B, H, T * 64, 128)
