// spb_head_layout.h -- how the lm head tiles its work (shared by the host
// planner, which sizes workspaces, and the launcher).
#pragma once

namespace spb {

inline int n_vocab_slices(int vocab) { return (vocab + 255) / 256; }
// bf16 planes of a gathered hidden row: three (hi, mid, lo) for the fp32 head
inline int head_planes(int kind) { return kind == 2 ? 3 : 1; }

// Scored rows per lm-head work group: n_chunks chunks of 32*mb rows (mb in
// 1..8), the fewest chunks of at most 256 rows, each as small as possible.
inline void head_m_layout(int M, int *n_chunks, int *mb) {
  int n = (M + 255) / 256;
  if (n < 1) n = 1;
  int per = (M + n - 1) / n;
  int b = (per + 31) / 32;
  *n_chunks = n;
  *mb = b < 1 ? 1 : (b > 8 ? 8 : b);
}

}  // namespace spb
