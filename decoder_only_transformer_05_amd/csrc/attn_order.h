// attn_order.h -- workgroup order of the attention dK/dV grids (attention.hip and
// attention_bf16.hip): one workgroup per block of nkb key blocks of one (batch, head).
#pragma once

#include "common.h"

namespace gpt2 {

// XCD-local (as xcd_logical_block), and inside each XCD's share all first key blocks (the
// most query tiles under the causal mask) before all second ones, and so on, so the longest
// blocks start first. Falls back to the plain XCD-local order when the grid does not split
// evenly.
GPT2_DEVICE_INLINE void key_block_of(int nkb, int NH, int* kb, int* head, int* b) {
  const int n = gridDim.x;
  const int per = n >> 3;
  int bh, k;
  if ((n & 7) == 0 && per % nkb == 0) {
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int groups = per / nkb;  // (batch, head) pairs on this XCD
    k = idx / groups;
    bh = xcd * groups + idx % groups;
  } else {
    const int lid = xcd_logical_block(blockIdx.x, n);
    k = lid % nkb;
    bh = lid / nkb;
  }
  *kb = k;
  *head = bh % NH;
  *b = bh / NH;
}

}  // namespace gpt2
