// Arguments of the chunked persistent forward pipeline (see pipeline.hip).
#pragma once
#include "common.h"

namespace moe {

struct PipeArgs {
  int T, D, I, E, K, Is;
  int n;           // routed slots
  int b;           // chunk rows (multiple of 256)
  int C;           // chunks
  int S;           // ring stages
  int ntn1, ntn2, ntn_s1, ntn_s2, sh_mt;       // n-tiles of the GEMMs, m-tiles of the shared expert
  int n_sh1, n_sh2, d_pre;                     // item counts: shared up/gate, shared down, dispatch prefix
  const uint16_t* x;
  const int32_t* perm;
  const int32_t* offsets;
  const uint16_t *wg, *wu, *wd, *sg, *su, *sd;
  uint16_t *x_ring, *h_ring, *y, *sh_h, *sh_out;
  const int32_t* ctile;       // [C][E+1] m-tile prefix of each chunk over experts
  const int32_t* chunk_base;  // [C+1] first item of each chunk's block
  int32_t* ctr;               // [0] ticket, [1] shared up/gate done, then dcnt[C], g1cnt[C], g2cnt[C]
  int32_t* err;
};

}  // namespace moe
