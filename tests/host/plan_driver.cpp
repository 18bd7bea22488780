// Host-logic driver for the sanitizer test: reads shapes (one per line: T D E
// F k F_shared has_router_bias expert_begin num_local_experts weight_format)
// and prints, per shape, the codes and sizes of the workspace planners, after
// checking that every planned region is 256-byte aligned, in order and inside
// the total.
#include <cstdio>

#include "plan.hpp"

static bool ordered(const size_t* off, int n, size_t total) {
  for (int i = 0; i < n; ++i) {
    if (off[i] % 256) return false;
    if (i && off[i] < off[i - 1]) return false;
    if (off[i] > total) return false;
  }
  return true;
}

int main() {
  moe_shape s;
  while (std::scanf("%d %d %d %d %d %d %d %d %d %d", &s.T, &s.D, &s.E, &s.F, &s.k, &s.F_shared,
                    &s.has_router_bias, &s.expert_begin, &s.num_local_experts,
                    &s.weight_format) == 10) {
    moe::Plan P;
    const int rc = moe::make_plan(&s, &P);
    if (rc != moe::check_shape(&s)) return 2;
    if (rc) {
      std::printf("%d\n", rc);
      continue;
    }
    const size_t off[] = {P.off_ids,      P.off_w,       P.off_counts,  P.off_offsets,
                          P.off_padded,   P.off_ntiles,  P.off_sorted,  P.off_rowof,
                          P.off_rowtoken, P.off_tilegroup, P.off_h,     P.off_yp,
                          P.off_partial,  P.off_rpart};
    if (!ordered(off, 14, P.total)) return 3;
    moe::BwdPlan B;
    const int rb = moe::make_backward_plan(&s, &B);
    size_t btotal = 0;
    if (!rb) {
      const size_t boff[] = {P.total,   B.off_rowa, B.off_xr, B.off_dyr, B.off_gu, B.off_dhp,
                             B.off_dgu, B.off_dp,   B.off_dl, B.off_pdy, B.off_hr};
      if (!ordered(boff, 11, B.total)) return 4;
      btotal = B.total;
    }
    std::printf("%d %d %zu %d %zu\n", rc, moe::choose_block_m(&s), P.total, rb, btotal);
  }
  return 0;
}
